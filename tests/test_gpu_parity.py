"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs.

Gates (tests/gates.py): fp32 normwise relative error <= 1e-5; bf16 KV max
absolute error <= 1e-2 and normwise <= 1e-3; lse within 1e-5 / 1e-4
relative; the cache append bit-exact.  Small cases compare every element;
full-size workloads compare sampled (b, h) rows (the oracle computes them
one by one) plus every appended cache row.
"""
import dataclasses

import numpy as np
import pytest
import torch

import kv_cache_gqa_decode_amd as kvd
from kv_cache_gqa_decode_amd import workloads as W
from tests import gates
from tests.gpu_helpers import (appended_rows, assert_q_rot, bits, device, gpu_step, opts,
                               oracle_step, upload)

pytestmark = pytest.mark.gpu


def check_full(p: W.Problem, kernel=None, split=0, style="interleaved", what="", tail=(0, -1),
               order=None):
    """Every output element and every cache element against the oracle."""
    dev = device()
    s = p.spec
    t = upload(p, dev)
    q_rot, out, lse = gpu_step(t, s, p.max_len, style=style,
                               options=opts(kernel, split, tail, order))
    oq, oo, ol, okc, ovc = oracle_step(p, style=style)
    kc, vc = W.from_torch(t["k_cache"]), W.from_torch(t["v_cache"])
    assert np.array_equal(bits(kc), bits(okc)), f"{what}: K cache differs from the oracle's"
    assert np.array_equal(bits(vc), bits(ovc)), f"{what}: V cache differs from the oracle's"
    qr = q_rot.cpu().numpy()
    assert_q_rot(qr, oq, what)
    e = gates.assert_out(out.cpu().numpy(), oo, s.dtype, what)
    gates.assert_lse(lse.cpu().numpy(), ol, s.dtype, what)
    return e


# ------------------------------------------------------- the small workloads

@pytest.mark.parametrize("style", ["interleaved", "half"])
def test_c1_fp32_single_step(style):
    p = W.make_problem(W.spec("c1"))
    check_full(p, style=style, what=f"c1 {style}")


@pytest.mark.parametrize("q_gain", [1.0, 32.0])
def test_c2_bf16_llama_shape(q_gain):
    p = W.make_problem(W.spec("c2", q_gain=q_gain))
    check_full(p, what=f"c2 q_gain={q_gain}")


# --------------------------------------------- ragged, split and paged cases

RAGGED = np.array([1, 2, 15, 16, 17, 63, 64, 65, 300, 1000, 1023, 1024], np.int32)


KERNELS = [("f32", "valu"), ("bf16", "valu"), ("bf16", "mfma")]


@pytest.mark.parametrize("dtype,kernel", KERNELS)
@pytest.mark.parametrize("split", [0, 16, 64, 208])
def test_varlen_contiguous(dtype, kernel, split):
    s = W.spec("c3", batch=RAGGED.size, max_seq_len=1024, dtype=dtype, q_gain=8.0)
    p = W.make_problem(s, lengths=RAGGED)
    check_full(p, kernel=kernel, split=split, what=f"varlen {dtype} {kernel} split={split}")


@pytest.mark.parametrize("kernel", ["valu", "mfma"])
@pytest.mark.parametrize("split", [0, 16, 48, 256])
@pytest.mark.parametrize("block_size", [16, 32])
def test_paged_small(kernel, split, block_size):
    s = W.spec("c4", batch=RAGGED.size, num_blocks=16000 // block_size,
               max_blocks_per_seq=1024 // block_size, block_size=block_size, q_gain=8.0)
    p = W.make_problem(s, lengths=RAGGED)
    check_full(p, kernel=kernel, split=split, what=f"paged{block_size} {kernel} split={split}")


def shared_prefix(p: W.Problem, n_shared: int) -> W.Problem:
    """The rows of every sequence whose append lands past the first n_shared
    blocks start with the first n_shared blocks of the longest sequence (a
    shared prompt prefix, read only: appends stay in private blocks)."""
    t = p.block_table.copy()
    src = int(np.argmax(p.positions))
    share = p.positions // p.spec.block_size >= n_shared
    share[src] = False
    t[share, :n_shared] = t[src, :n_shared]
    assert share.sum() >= 2
    return dataclasses.replace(p, block_table=t)


@pytest.mark.parametrize("kernel", ["valu", "mfma"])
@pytest.mark.parametrize("block_size", [16, 32])
@pytest.mark.parametrize("split", [0, 48])
def test_shared_prefix_blocks(kernel, block_size, split):
    s = W.spec("c4", batch=RAGGED.size, num_blocks=16000 // block_size,
               max_blocks_per_seq=1024 // block_size, block_size=block_size, q_gain=8.0)
    p = shared_prefix(W.make_problem(s, lengths=RAGGED), 128 // block_size)
    check_full(p, kernel=kernel, split=split, what=f"shared prefix {block_size} {kernel}")


def test_auto_plan_picks_matrix_cores_for_bf16():
    dev = device()
    k = torch.empty((4, 64, 8, 128), dtype=torch.bfloat16, device=dev)
    assert kvd.get_plan(4, 32, k)["kernel"] == "mfma"
    assert kvd.get_plan(4, 8 * 64, k)["kernel"] == "valu"          # n_rep 64
    k32 = torch.empty((4, 64, 8, 128), dtype=torch.float32, device=dev)
    assert kvd.get_plan(4, 32, k32)["kernel"] == "valu"
    with pytest.raises(kvd.KvdError):
        kvd.get_plan(4, 32, k32, options=kvd.Options(kernel="mfma"))


@pytest.mark.parametrize("kernel", ["valu", "mfma"])
@pytest.mark.parametrize("split", [0, 32])
@pytest.mark.parametrize("block_size", [16, 32])
def test_paged_equals_contiguous_bitwise(kernel, split, block_size):
    """The same logical cache, paged or contiguous, gives identical bits."""
    dev = device()
    L = np.array([5, 16, 333, 1024, 700], np.int32)
    sp = W.spec("c4", batch=5, num_blocks=8000 // block_size, max_blocks_per_seq=1024 // block_size,
                block_size=block_size)
    sc = W.spec("c3", batch=5, max_seq_len=1024).replace(cfg_id=sp.cfg_id)
    res = []
    for s in (sp, sc):
        p = W.make_problem(s, lengths=L)
        t = upload(p, dev)
        q_rot, out, lse = gpu_step(t, s, 1024, options=opts(kernel, split))
        res.append((q_rot.cpu(), out.cpu(), lse.cpu()))
    for a, b in zip(res[0], res[1]):
        assert torch.equal(a, b)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype,kernel", KERNELS)
@pytest.mark.parametrize("n_rep", [1, 2, 4, 8, 16, 32])
def test_gqa_ratios(D, dtype, kernel, n_rep):
    H = 32
    G = H // n_rep
    L = np.array([700, 129, 1], np.int32)
    s = W.spec("c3", batch=3, n_heads=H, n_kv_heads=G, head_dim=D, max_seq_len=768,
               dtype=dtype, q_gain=4.0, value_scale=D ** -0.5 if dtype == "bf16" else 1.0)
    p = W.make_problem(s, lengths=L)
    check_full(p, kernel=kernel, what=f"D={D} {dtype} {kernel} n_rep={n_rep}")


def test_zero_lengths_and_empty_bound():
    dev = device()
    s = W.spec("c3", batch=3, max_seq_len=64)
    p = W.make_problem(s, lengths=np.array([3, 10, 64], np.int32))
    t = upload(p, dev)
    q_rot = kvd.rope_append_kv(t["q"], t["k_new"], t["v_new"], t["k_cache"], t["v_cache"],
                               t["positions"])
    lens = torch.tensor([0, 10, 0], dtype=torch.int32, device=dev)
    out, lse = kvd.gqa_decode_attn(q_rot, t["k_cache"], t["v_cache"], lens, max_seq_len=64)
    torch.cuda.synchronize()
    assert (out[0] == 0).all() and (out[2] == 0).all()
    assert torch.isinf(lse[0]).all() and (lse[0] < 0).all()
    assert torch.isfinite(out[1]).all()
    # a zero host bound: nothing can be attended
    out, lse = kvd.gqa_decode_attn(q_rot, t["k_cache"], t["v_cache"], lens * 0, max_seq_len=0)
    torch.cuda.synchronize()
    assert (out == 0).all() and torch.isinf(lse).all()


def test_out_of_range_positions_skip_the_append():
    """Positions the host cannot check (device-resident): the kernel leaves
    the cache untouched instead of writing out of bounds."""
    dev = device()
    s = W.spec("c3", batch=3, max_seq_len=64)
    p = W.make_problem(s, lengths=np.array([3, 10, 64], np.int32))
    t = upload(p, dev)
    before = t["k_cache"].clone()
    bad = torch.tensor([-1, 64, 1 << 30], dtype=torch.int32, device=dev)
    kvd.rope_append_kv(t["q"], t["k_new"], t["v_new"], t["k_cache"], t["v_cache"], bad)
    torch.cuda.synchronize()
    assert torch.equal(before.view(torch.int16), t["k_cache"].view(torch.int16))


@pytest.mark.parametrize("kernel", ["valu", "mfma"])
def test_split_counts_agree(kernel):
    """Different split sizes reduce in different orders: results agree to
    rounding and every one matches the oracle."""
    s = W.spec("c3", batch=2, max_seq_len=4096, q_gain=16.0)
    p = W.make_problem(s, lengths=np.array([4096, 2500], np.int32))
    for split in (16, 128, 1024, 4096):
        check_full(p, kernel=kernel, split=split, what=f"{kernel} split={split}")


def test_workspace_too_small_is_reported():
    dev = device()
    s = W.spec("c3", batch=2, max_seq_len=2048)
    p = W.make_problem(s, lengths=np.array([2048, 100], np.int32))
    t = upload(p, dev)
    o = kvd.Options(split_tokens=64)
    q_rot = kvd.rope_append_kv(t["q"], t["k_new"], t["v_new"], t["k_cache"], t["v_cache"],
                               t["positions"])
    need = kvd.workspace_size(q_rot, t["k_cache"], max_seq_len=2048, options=o)
    assert need > kvd.workspace_size(q_rot, t["k_cache"], max_seq_len=2048,
                                     options=kvd.Options(split_tokens=1024)) > 0
    small = torch.empty(need - 256, dtype=torch.uint8, device=dev)
    with pytest.raises(kvd.KvdError) as ei:
        kvd.gqa_decode_attn(q_rot, t["k_cache"], t["v_cache"], t["seq_lens"], max_seq_len=2048,
                            workspace=small, options=o)
    assert ei.value.status == 4


def test_repeated_steps_are_idempotent():
    """Re-running the step at the same positions rewrites the same bits and
    gives the same outputs (what the benchmark's timed loop relies on)."""
    dev = device()
    s = W.spec("c3", batch=4, max_seq_len=512)
    p = W.make_problem(s, lengths=np.array([512, 77, 300, 1], np.int32))
    t = upload(p, dev)
    first = [x.clone() for x in gpu_step(t, s, 512)]
    k1 = t["k_cache"].clone()
    for _ in range(3):
        again = gpu_step(t, s, 512)
    for a, b in zip(first, again):
        assert torch.equal(a, b)
    assert torch.equal(k1.view(torch.int16), t["k_cache"].view(torch.int16))


@pytest.mark.parametrize("kernel", ["valu", "mfma"])
@pytest.mark.parametrize("split,tail,span", [(256, 64, 400), (512, 128, 1024), (128, 16, 96),
                                             (1024, 1024, 500), (256, 32, 0)])
@pytest.mark.parametrize("order", [None, 0, 1, 2, 3, 4])
def test_two_level_splits(kernel, split, tail, span, order):
    """Splits of `split` tokens, then of `tail` tokens over the last `span`
    positions of the bound, in every dispatch order: the merge sees the same
    result as one softmax over the sequence."""
    if kernel == "valu" and order is not None:
        pytest.skip("the VALU kernel has one dispatch order")
    s = W.spec("c3", batch=RAGGED.size, max_seq_len=1024, q_gain=8.0)
    p = W.make_problem(s, lengths=RAGGED)
    check_full(p, kernel=kernel, split=split, tail=(tail, span), order=order,
               what=f"{kernel} split={split} tail={tail}/{span} order={order}")


@pytest.mark.parametrize("kernel", ["mfma"])
@pytest.mark.parametrize("order", [0, 1, 2, 3, 4])
def test_two_level_splits_paged(kernel, order):
    s = W.spec("c4", batch=RAGGED.size, num_blocks=1000, max_blocks_per_seq=64, q_gain=8.0)
    p = W.make_problem(s, lengths=RAGGED)
    check_full(p, kernel=kernel, split=256, tail=(32, 300), order=order,
               what=f"paged {kernel} two-level order={order}")


@pytest.mark.parametrize("kernel", ["valu", "mfma"])
@pytest.mark.parametrize("order", [None, 1, 3, 4])
def test_empty_sequences_with_several_splits(kernel, order):
    """Zero-length sequences among long ones with several splits: the work
    list holds no unit for them, the merge still writes out = 0, lse = -inf,
    and the others match the oracle."""
    if kernel == "valu" and order is not None:
        pytest.skip("the VALU kernel has one dispatch order")
    dev = device()
    s = W.spec("c3", batch=5, max_seq_len=1024, q_gain=8.0)
    p = W.make_problem(s, lengths=np.array([1, 300, 1, 1024, 17], np.int32))
    t = upload(p, dev)
    q_rot = kvd.rope_append_kv(t["q"], t["k_new"], t["v_new"], t["k_cache"], t["v_cache"],
                               t["positions"])
    lens = torch.tensor([0, 300, 0, 1024, 17], dtype=torch.int32, device=dev)
    out, lse = kvd.gqa_decode_attn(q_rot, t["k_cache"], t["v_cache"], lens, max_seq_len=1024,
                                   options=opts(kernel, 64, order=order))
    torch.cuda.synchronize()
    assert (out[0] == 0).all() and (out[2] == 0).all()
    assert torch.isinf(lse[0]).all() and torch.isinf(lse[2]).all()
    p.seq_lens[:] = [0, 300, 0, 1024, 17]
    oq, oo, ol, _, _ = oracle_step(p)
    keep = [1, 3, 4]
    gates.assert_out(out.cpu().numpy()[keep], oo[keep], "bf16", "empty sequences")
    gates.assert_lse(lse.cpu().numpy()[keep], ol[keep], "bf16", "empty sequences")


@pytest.mark.parametrize("dtype", ["bf16", "i8"])
@pytest.mark.parametrize("batch", [64, 65, 2])
def test_work_list_derived_in_kernel(dtype, batch):
    """Dispatch order 4 (each wave derives its unit from the lengths, up to 64
    sequences) against order 3 (the list built by its own launch): a batch
    whose partial last splits tie in every 16-token bucket, with empty
    sequences, lengths below one bucket and exact multiples of the split,
    and a NaN-filled workspace, so a unit that no workgroup computed would
    surface as NaN.  The two orders give the same bits, and the oracle's
    result.  65 sequences exceed the lanes of a wave: order 4 then falls
    back to order 3."""
    dev = device()
    rng = np.random.default_rng(batch)
    base = np.array([0, 1, 5, 16, 17, 31, 32, 100, 111, 256, 257, 511, 512, 513, 700, 1024],
                    np.int32)
    lens = np.resize(base, batch).copy()
    rng.shuffle(lens)
    lens[lens == 0] = 1                      # the append needs a slot; emptied below
    s = W.spec("c3", batch=batch, max_seq_len=1024, q_gain=8.0).replace(dtype=dtype)
    p = W.make_problem(s, lengths=lens)
    t = upload(p, dev)
    q_rot = gpu_step(t, s, 1024)[0]
    empty = np.flatnonzero(np.resize(base, batch) == 0)
    run_lens = lens.copy()
    run_lens[empty] = 0
    lens_t = torch.tensor(run_lens, dtype=torch.int32, device=dev)
    results = []
    for order in (3, 4):
        o = kvd.Options(split_tokens=128, dispatch_order=order)
        nbytes = kvd.workspace_size(q_rot, t["k_cache"], max_seq_len=1024, options=o)
        ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device=dev)
        if dtype == "i8":
            out, lse = kvd.gqa_decode_attn_int8(q_rot, t["k_cache"], t["v_cache"], t["k_scale"],
                                                t["v_scale"], lens_t, max_seq_len=1024,
                                                workspace=ws, options=o)
        else:
            out, lse = kvd.gqa_decode_attn(q_rot, t["k_cache"], t["v_cache"], lens_t,
                                           max_seq_len=1024, workspace=ws, options=o)
        torch.cuda.synchronize()
        results.append((out.clone(), lse.clone()))
    assert torch.equal(results[0][0], results[1][0]), "orders 3 and 4 differ"
    assert torch.equal(results[0][1], results[1][1]), "orders 3 and 4 differ (lse)"
    out, lse = (x.cpu().numpy() for x in results[1])
    assert (out[empty] == 0).all() and np.isneginf(lse[empty]).all()
    p.seq_lens[:] = run_lens
    _, oo, ol, _, _ = oracle_step(p)
    keep = np.flatnonzero(run_lens > 0)
    gates.assert_out(out[keep], oo[keep], dtype, f"work list order 4, B={batch}")
    gates.assert_lse(lse[keep], ol[keep], dtype, f"work list order 4, B={batch}")


@pytest.mark.parametrize("dtype,kernel", KERNELS)
@pytest.mark.parametrize("D,batch,split", [(128, 1027, 16), (64, 1025, 16), (128, 1027, 128)])
def test_merge_of_many_rows(dtype, kernel, D, batch, split):
    """Over a thousand query rows (one head per sequence, a row count that is
    not a multiple of 4) with 1 to 64 splits per sequence: the merge takes
    a wave per row, four rows to a workgroup, the last workgroup partly
    empty, and split lanes that run several batches of loads."""
    rng = np.random.default_rng(batch + D + split)
    L = rng.integers(1, 1025, batch).astype(np.int32)
    L[:5] = [1, 1024, 16, 17, 1023]
    s = W.spec("c3", batch=batch, n_heads=1, n_kv_heads=1, head_dim=D, max_seq_len=1024,
               dtype=dtype, q_gain=4.0, value_scale=D ** -0.5 if dtype == "bf16" else 1.0)
    p = W.make_problem(s, lengths=L)
    check_full(p, kernel=kernel, split=split, what=f"{dtype} {kernel} D={D} B={batch} split={split}")


# --------------------------- reachable paths: long splits, bad table entries

LONG = np.array([8192, 7001, 6150, 4097, 300], np.int32)


@pytest.mark.parametrize("kernel", ["valu", "mfma"])
@pytest.mark.parametrize("block_size", [16, 32])
@pytest.mark.parametrize("split", [6144, 8192])
def test_paged_long_splits(kernel, block_size, split):
    """Splits above 4096 tokens: a wave of the matrix-core kernel then holds
    the ids of the blocks it visits in a second register."""
    s = W.spec("c4", batch=LONG.size, num_blocks=48000 // block_size,
               max_blocks_per_seq=8192 // block_size, block_size=block_size, q_gain=8.0)
    p = W.make_problem(s, lengths=LONG)
    check_full(p, kernel=kernel, split=split, what=f"paged{block_size} {kernel} split={split}")


def bad_table(p: W.Problem):
    """The problem's table with entries outside the pool: two inside the
    history of sequence 9, the appended block of sequences 10 and 4 (their
    appends must be skipped) and the first block of sequence 10.  Returns
    (table, the sequences left intact, the sequences whose append lands)."""
    s = p.spec
    bs = s.block_size
    t = p.block_table.copy()
    t[9, 5] = -1
    t[9, 20] = s.num_blocks + 7
    for b, v in ((10, -5), (4, s.num_blocks)):
        t[b, int(p.positions[b]) // bs] = v
    t[10, 0] = 2 ** 31 - 1
    intact = [b for b in range(s.batch) if b not in (4, 9, 10)]
    appended = [b for b in range(s.batch) if b not in (4, 10)]
    return t, intact, appended


def _subset(p: W.Problem, rows):
    s = p.spec
    return dataclasses.replace(
        p, spec=s.replace(batch=len(rows)), q=p.q[rows], k_new=p.k_new[rows],
        v_new=p.v_new[rows], positions=p.positions[rows], seq_lens=p.seq_lens[rows],
        block_table=p.block_table[rows])


def run_bad_table(p: W.Problem, options):
    """GPU step on a table with out-of-pool entries: the intact sequences
    equal the oracle, every output is finite or (no valid token) 0 / -inf,
    and the caches equal the oracle's after the appends whose block is in
    the pool (no write through a bad id)."""
    dev = device()
    s = p.spec
    table, intact, appended = bad_table(p)
    t = upload(p, dev)
    t["block_table"] = W.as_torch(table, dev)
    q_rot, out, lse = gpu_step(t, s, p.max_len, options=options)
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    assert np.isfinite(out).all()
    assert not np.isnan(lse).any()
    _, oo, ol, _, _ = oracle_step(_subset(p, intact))
    gates.assert_out(out[intact], oo, s.dtype, "intact sequences")
    gates.assert_lse(lse[intact], ol, s.dtype, "intact sequences")
    _, _, _, okc, ovc = oracle_step(_subset(p, appended))
    assert np.array_equal(bits(W.from_torch(t["k_cache"])), bits(okc)), "K pool differs"
    assert np.array_equal(bits(W.from_torch(t["v_cache"])), bits(ovc)), "V pool differs"


@pytest.mark.parametrize("kernel", ["valu", "mfma"])
@pytest.mark.parametrize("block_size", [16, 32])
@pytest.mark.parametrize("split", [0, 48])
def test_block_ids_outside_the_pool(kernel, block_size, split):
    s = W.spec("c4", batch=RAGGED.size, num_blocks=16000 // block_size,
               max_blocks_per_seq=1024 // block_size, block_size=block_size, q_gain=8.0)
    run_bad_table(W.make_problem(s, lengths=RAGGED), opts(kernel, split))


# ------------------------------------------------- streams and timing events

def test_two_streams_concurrently():
    """Two decode steps enqueued on two streams at once, each with the
    workspace the binding allocates per call on its stream: both equal the
    oracle (a workspace shared across streams would mix their partials)."""
    dev = device()
    probs = []
    for i, (B, L) in enumerate([(16, 4096), (24, 2048)]):
        s = W.spec("c3", batch=B, max_seq_len=L, len_lo=L // 4, len_hi=L, q_gain=8.0)
        s = s.replace(cfg_id=s.cfg_id + 100 * (i + 1))
        p = W.make_problem(s)
        probs.append((s, p, upload(p, dev)))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(dev), torch.cuda.Stream(dev)]
    res = [None, None]
    for _ in range(4):
        for i, ((s, p, t), st) in enumerate(zip(probs, streams)):
            st.wait_stream(torch.cuda.current_stream(dev))
            with torch.cuda.stream(st):
                res[i] = gpu_step(t, s, p.max_len, sync=False)
    torch.cuda.synchronize()
    for (s, p, t), (q_rot, out, lse) in zip(probs, res):
        _, oo, ol, _, _ = oracle_step(p)
        gates.assert_out(out.cpu().numpy(), oo, s.dtype, f"stream B={s.batch}")
        gates.assert_lse(lse.cpu().numpy(), ol, s.dtype, f"stream B={s.batch}")


def test_option_events_bracket_the_split_kernel():
    """Events passed in the options are recorded around the split kernel:
    their interval is positive and inside the whole call's."""
    dev = device()
    s = W.spec("c3", batch=8, max_seq_len=4096, len_lo=2048, len_hi=4096)
    p = W.make_problem(s)
    t = upload(p, dev)
    q_rot = gpu_step(t, s, p.max_len)[0]
    e0, e1, a, b = (torch.cuda.Event(enable_timing=True) for _ in range(4))
    a.record()
    kvd.gqa_decode_attn(q_rot, t["k_cache"], t["v_cache"], t["seq_lens"], max_seq_len=p.max_len,
                        options=kvd.Options(events=(e0, e1)))
    b.record()
    torch.cuda.synchronize()
    k_ms, all_ms = e0.elapsed_time(e1), a.elapsed_time(b)
    assert 0 < k_ms <= all_ms
