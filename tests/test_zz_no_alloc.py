"""gqa_decode_attn_multi_noalloc, the entry point for callers that cannot
allocate device memory, through the C ABI: the same bits as
gqa_decode_attn_multi with a caller workspace, on two calls in a row (the
second on a smaller problem, so stale partials of the first sit in the
library's array), the oracle's result within the gates, no device memory
taken by repeated calls, and a refusal when the split partials would exceed
the array."""
import numpy as np
import pytest
import torch

import kv_cache_gqa_decode_amd as kvd
from kv_cache_gqa_decode_amd import _binding as B
from kv_cache_gqa_decode_amd import workloads as W
from tests import gates
from tests.gpu_helpers import device, upload
from tests.test_gpu_multi import oracle_window

pytestmark = pytest.mark.gpu


def _bits(x):
    return x.contiguous().view(torch.int32)


def _problem(dtype, paged, B_, L_hi, T, seed):
    if paged:
        s = W.spec("c4", batch=B_, num_blocks=B_ * (L_hi // 16) + 16,
                   max_blocks_per_seq=L_hi // 16, len_lo=T, len_hi=L_hi, q_gain=8.0)
    else:
        s = W.spec("c3", batch=B_, max_seq_len=L_hi, len_lo=T, len_hi=L_hi, q_gain=8.0)
    s = s.replace(dtype=dtype, cfg_id=s.cfg_id + seed)
    return s, W.make_window(s, T)


def _run(dev, s, p, options=None):
    t = upload(p, dev)
    sc = dict(k_scale=t["k_scale"], v_scale=t["v_scale"]) if s.dtype == "i8" else {}
    q_rot = kvd.rope_append_kv_multi(t["q"], t["k_new"], t["v_new"], t["k_cache"], t["v_cache"],
                                     t["positions"], t["block_table"], base=s.rope_base, **sc)
    ref_out, ref_lse = kvd.gqa_decode_attn_multi(q_rot, t["k_cache"], t["v_cache"], t["seq_lens"],
                                                 t["block_table"], max_seq_len=p.max_len,
                                                 options=options, **sc)
    out = torch.full_like(ref_out, float("nan"))
    lse = torch.full_like(ref_lse, float("nan"))
    kvd.gqa_decode_attn_noalloc(q_rot, t["k_cache"], t["v_cache"], t["seq_lens"],
                                t["block_table"], max_seq_len=p.max_len, out=out, lse=lse,
                                options=options, **sc)
    torch.cuda.synchronize()
    return t, q_rot, ref_out, ref_lse, out, lse, sc


@pytest.mark.parametrize("dtype,paged,T", [("bf16", False, 1), ("bf16", True, 5),
                                           ("i8", True, 1), ("i8", False, 5)])
def test_noalloc_equals_workspace_call_twice(dtype, paged, T):
    dev = device()
    gd = "i8" if dtype == "i8" else "bf16"
    for B_, L_hi, seed in ((24, 4096, 0), (3, 640, 7)):       # the second call is smaller
        s, p = _problem(dtype, paged, B_, L_hi, T, seed)
        print(f"[noalloc] {dtype} paged={paged} T={T} B={B_} L<={L_hi}", flush=True)
        t, q_rot, ref_out, ref_lse, out, lse, _ = _run(dev, s, p)
        assert torch.equal(_bits(out), _bits(ref_out)), "out differs from the workspace call"
        assert torch.equal(_bits(lse), _bits(ref_lse)), "lse differs from the workspace call"
        _, oo, ol, _, _ = oracle_window(p)
        gates.assert_out(out.cpu().numpy(), oo, gd, f"noalloc B={B_}")
        gates.assert_lse(lse.cpu().numpy(), ol, gd, f"noalloc B={B_}")


def test_noalloc_takes_no_device_memory():
    dev = device()
    s, p = _problem("bf16", False, 16, 4096, 1, 3)
    t, q_rot, ref_out, ref_lse, out, lse, _ = _run(dev, s, p)     # first call: array looked up
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info(dev)[0]
    for _ in range(20):
        kvd.gqa_decode_attn_noalloc(q_rot, t["k_cache"], t["v_cache"], t["seq_lens"],
                                    max_seq_len=p.max_len, out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info(dev)[0] == free0
    assert torch.equal(_bits(out), _bits(ref_out))


def test_noalloc_refuses_partials_beyond_the_array():
    """16-token splits over up to 8192 positions for 6 sequences: about
    6 * 32 * 500 split rows of 129 floats, ~50 MB > 32 MiB; the workspace
    call takes them."""
    dev = device()
    s, p = _problem("bf16", False, 6, 8192, 1, 11)
    o = kvd.Options(split_tokens=16)
    t = upload(p, dev)
    q_rot = kvd.rope_append_kv_multi(t["q"], t["k_new"], t["v_new"], t["k_cache"], t["v_cache"],
                                     t["positions"])
    assert kvd.workspace_size(q_rot, t["k_cache"], None, p.max_len, n_query=1,
                              options=o) > B.NOALLOC_SCRATCH_BYTES
    with pytest.raises(kvd.KvdError) as ei:
        kvd.gqa_decode_attn_noalloc(q_rot, t["k_cache"], t["v_cache"], t["seq_lens"],
                                    max_seq_len=p.max_len, options=o)
    assert ei.value.status == 4
    out, lse = kvd.gqa_decode_attn_multi(q_rot, t["k_cache"], t["v_cache"], t["seq_lens"],
                                         max_seq_len=p.max_len, options=o)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
