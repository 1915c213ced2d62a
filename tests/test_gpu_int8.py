"""GPU parity of the INT8 KV cache: rope_append_kv_int8 and
gqa_decode_attn_int8 through the C ABI against the fp64 oracle on the same
seeded codes and scales.

The stored codes must be bit-exact (both sides quantise the exact rotated
key and v_new with an fp64 quotient, ties to even); outputs pass the bf16
gates (both sides dequantise the same codes, so only arithmetic differs).
Every case compares every output row and lse, and both caches in full.
"""
import numpy as np
import pytest
import torch

import kv_cache_gqa_decode_amd as kvd
from kv_cache_gqa_decode_amd import workloads as W
from tests import gates
from tests.gpu_helpers import assert_q_rot, device, gpu_step, opts, oracle_step, upload
from tests.test_gpu_parity import shared_prefix

pytestmark = pytest.mark.gpu

RAGGED = np.array([1, 2, 15, 16, 17, 63, 64, 65, 300, 1000, 1023, 1024], np.int32)


def i8(name, **kw):
    return W.spec(name, **kw).replace(dtype="i8")


def check_full(p: W.Problem, split=0, style="interleaved", what="", tail=(0, -1), order=None):
    dev = device()
    s = p.spec
    t = upload(p, dev)
    q_rot, out, lse = gpu_step(t, s, p.max_len, style=style,
                               options=opts(None, split, tail, order))
    oq, oo, ol, okc, ovc = oracle_step(p, style=style)
    assert np.array_equal(W.from_torch(t["k_cache"]), okc), f"{what}: K codes differ"
    assert np.array_equal(W.from_torch(t["v_cache"]), ovc), f"{what}: V codes differ"
    qr = q_rot.cpu().numpy()
    assert_q_rot(qr, oq, what)
    e = gates.assert_out(out.cpu().numpy(), oo, "i8", what)
    gates.assert_lse(lse.cpu().numpy(), ol, "i8", what)
    return e


@pytest.mark.parametrize("q_gain", [1.0, 32.0])
def test_llama_shape_context_1024(q_gain):
    p = W.make_problem(i8("c2", q_gain=q_gain))
    check_full(p, what=f"int8 c2 q_gain={q_gain}")


@pytest.mark.parametrize("style", ["interleaved", "half"])
def test_rope_styles(style):
    p = W.make_problem(i8("c3", batch=3, max_seq_len=256, q_gain=4.0),
                       lengths=np.array([1, 100, 256], np.int32))
    check_full(p, style=style, what=f"int8 {style}")


@pytest.mark.parametrize("split", [0, 16, 64, 208, 256])
def test_varlen_contiguous(split):
    s = i8("c3", batch=RAGGED.size, max_seq_len=1024, q_gain=8.0)
    check_full(W.make_problem(s, lengths=RAGGED), split=split, what=f"int8 varlen split={split}")


@pytest.mark.parametrize("split", [0, 16, 48, 256])
@pytest.mark.parametrize("block_size", [16, 32])
def test_paged_small(split, block_size):
    s = i8("c4", batch=RAGGED.size, num_blocks=16000 // block_size,
           max_blocks_per_seq=1024 // block_size, block_size=block_size, q_gain=8.0)
    check_full(W.make_problem(s, lengths=RAGGED), split=split,
               what=f"int8 paged{block_size} split={split}")


@pytest.mark.parametrize("block_size", [16, 32])
def test_shared_prefix_blocks(block_size):
    s = i8("c4", batch=RAGGED.size, num_blocks=16000 // block_size,
           max_blocks_per_seq=1024 // block_size, block_size=block_size, q_gain=8.0)
    p = shared_prefix(W.make_problem(s, lengths=RAGGED), 128 // block_size)
    check_full(p, split=48, what=f"int8 shared prefix {block_size}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("n_rep", [1, 2, 4, 8, 16, 32])
def test_gqa_ratios(D, n_rep):
    H = 32
    s = i8("c3", batch=3, n_heads=H, n_kv_heads=H // n_rep, head_dim=D, max_seq_len=768,
           q_gain=4.0, value_scale=D ** -0.5)
    p = W.make_problem(s, lengths=np.array([700, 129, 1], np.int32))
    check_full(p, what=f"int8 D={D} n_rep={n_rep}")


@pytest.mark.parametrize("split", [0, 32])
@pytest.mark.parametrize("block_size", [16, 32])
def test_paged_equals_contiguous_bitwise(split, block_size):
    dev = device()
    L = np.array([5, 16, 333, 1024, 700], np.int32)
    sp = i8("c4", batch=5, num_blocks=8000 // block_size, max_blocks_per_seq=1024 // block_size,
            block_size=block_size)
    sc = i8("c3", batch=5, max_seq_len=1024).replace(cfg_id=sp.cfg_id)
    res = []
    for s in (sp, sc):
        p = W.make_problem(s, lengths=L)
        t = upload(p, dev)
        res.append([x.cpu() for x in gpu_step(t, s, 1024, options=opts(None, split))])
    for a, b in zip(res[0], res[1]):
        assert torch.equal(a, b)


@pytest.mark.parametrize("block_size", [16, 32])
@pytest.mark.parametrize("split", [6144, 8192])
def test_paged_long_splits(block_size, split):
    """Splits above 4096 tokens (the block ids of a wave in a second register)."""
    L = np.array([8192, 7001, 6150, 4097, 300], np.int32)
    s = i8("c4", batch=L.size, num_blocks=48000 // block_size,
           max_blocks_per_seq=8192 // block_size, block_size=block_size, q_gain=8.0)
    check_full(W.make_problem(s, lengths=L), split=split,
               what=f"int8 paged{block_size} split={split}")


@pytest.mark.parametrize("block_size", [16, 32])
@pytest.mark.parametrize("split", [0, 64])
def test_block_ids_outside_the_pool(block_size, split):
    from tests.test_gpu_parity import run_bad_table
    s = i8("c4", batch=RAGGED.size, num_blocks=16000 // block_size,
           max_blocks_per_seq=1024 // block_size, block_size=block_size, q_gain=8.0)
    run_bad_table(W.make_problem(s, lengths=RAGGED), opts(None, split))


def test_split_counts_agree():
    s = i8("c3", batch=2, max_seq_len=4096, q_gain=16.0)
    p = W.make_problem(s, lengths=np.array([4096, 2500], np.int32))
    for split in (16, 256, 1024, 4096):
        check_full(p, split=split, what=f"int8 split={split}")


@pytest.mark.parametrize("split,tail,span", [(512, 128, 1024), (256, 32, 300)])
@pytest.mark.parametrize("order", [0, 1, 2, 3, 4])
def test_two_level_splits(split, tail, span, order):
    s = i8("c3", batch=RAGGED.size, max_seq_len=1024, q_gain=8.0)
    check_full(W.make_problem(s, lengths=RAGGED), split=split, tail=(tail, span), order=order,
               what=f"int8 split={split} tail={tail}/{span} order={order}")


def test_zero_lengths():
    dev = device()
    s = i8("c3", batch=3, max_seq_len=64)
    p = W.make_problem(s, lengths=np.array([3, 10, 64], np.int32))
    t = upload(p, dev)
    q_rot = kvd.rope_append_kv_int8(t["q"], t["k_new"], t["v_new"], t["k_cache"], t["v_cache"],
                                    t["k_scale"], t["v_scale"], t["positions"])
    lens = torch.tensor([0, 10, 0], dtype=torch.int32, device=dev)
    out, lse = kvd.gqa_decode_attn_int8(q_rot, t["k_cache"], t["v_cache"], t["k_scale"],
                                        t["v_scale"], lens, max_seq_len=64)
    torch.cuda.synchronize()
    assert (out[0] == 0).all() and (out[2] == 0).all()
    assert torch.isinf(lse[0]).all() and (lse[0] < 0).all()
    assert torch.isfinite(out[1]).all()


def test_repeated_steps_are_idempotent():
    dev = device()
    s = i8("c3", batch=4, max_seq_len=512)
    p = W.make_problem(s, lengths=np.array([512, 77, 300, 1], np.int32))
    t = upload(p, dev)
    first = [x.clone() for x in gpu_step(t, s, 512)]
    k1, v1 = t["k_cache"].clone(), t["v_cache"].clone()
    for _ in range(3):
        again = gpu_step(t, s, 512)
    for a, b in zip(first, again):
        assert torch.equal(a, b)
    assert torch.equal(k1, t["k_cache"]) and torch.equal(v1, t["v_cache"])


def test_plan_reports_the_int8_kernel():
    dev = device()
    k = torch.empty((4, 4, 8, 16, 128), dtype=torch.int8, device=dev)    # [B, S/16, G, 16, D]
    assert kvd.get_plan(4, 32, k)["kernel"] == "int8"
    with pytest.raises(kvd.KvdError):
        kvd.get_plan(4, 32, k, options=kvd.Options(kernel="mfma"))
    with pytest.raises(kvd.KvdError):
        kvd.get_plan(1, 64, torch.empty((1, 4, 1, 16, 128), dtype=torch.int8, device=dev))  # n_rep 64


# ------------------------------------------------------------- full sizes

def run_full_i8(s: W.Spec):
    dev = device()
    p = W.make_problem(s)
    print(f"[full int8] {s.name} G={s.n_kv_heads} B={s.batch} max_len={p.max_len}", flush=True)
    t = upload(p, dev)
    q_rot, out, lse = gpu_step(t, s, p.max_len)
    oq, oo, ol, okc, ovc = oracle_step(p)
    assert_q_rot(q_rot.cpu().numpy(), oq, f"int8 {s.name} q_rot")
    e = gates.assert_out(out.cpu().numpy(), oo, "i8", f"int8 {s.name} all rows")
    gates.assert_lse(lse.cpu().numpy(), ol, "i8", f"int8 {s.name} all rows lse")
    print(f"[full int8] {s.name} G={s.n_kv_heads}: {e}", flush=True)
    # both caches in full (the appended codes and everything else unchanged)
    assert torch.equal(t["k_cache"], torch.from_numpy(okc).to(dev))
    assert torch.equal(t["v_cache"], torch.from_numpy(ovc).to(dev))
    del t
    torch.cuda.empty_cache()


def test_c3_int8_full():
    run_full_i8(i8("c3"))


def test_c4_int8_full():
    run_full_i8(i8("c4"))


@pytest.mark.parametrize("G", [32, 8, 1])
def test_c5_int8_full(G):
    run_full_i8(i8("c5", n_kv_heads=G))
