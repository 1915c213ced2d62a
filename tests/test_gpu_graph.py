"""The decode step captured as one HIP graph (torch.cuda.graph around the
C-ABI calls) replays to the eager step's results, bit for bit.

The library's calls allocate nothing and record no memset, so a step can be
captured once and replayed; every replay is checked against the eager
result, with eager work of the program and synchronisations in between.
Both forms of the step: the two calls, and gqa_decode_step (one split-kernel
launch plus the merge; with T = 3 new tokens, gqa_decode_step_multi).
"""
import numpy as np
import pytest
import torch

import kv_cache_gqa_decode_amd as kvd
from kv_cache_gqa_decode_amd import workloads as W
from tests.gpu_helpers import device, upload

pytestmark = pytest.mark.gpu


def _bits(x):
    x = x.contiguous()
    return x.view({torch.bfloat16: torch.int16, torch.float32: torch.int32}.get(x.dtype, x.dtype))


def _step_fn(t, s, max_len, bufs, fused=False):
    q_rot, out, lse, ws = bufs
    i8 = s.dtype == "i8"

    def step():
        if fused:
            sc = dict(k_scale=t["k_scale"], v_scale=t["v_scale"]) if i8 else {}
            kvd.gqa_decode_step(t["q"], t["k_new"], t["v_new"], t["k_cache"], t["v_cache"],
                                t["positions"], t["block_table"], max_seq_len=max_len,
                                q_rot=q_rot, out=out, lse=lse, workspace=ws, **sc)
        elif i8:
            kvd.rope_append_kv_int8(t["q"], t["k_new"], t["v_new"], t["k_cache"], t["v_cache"],
                                    t["k_scale"], t["v_scale"], t["positions"], t["block_table"],
                                    q_rot=q_rot)
            kvd.gqa_decode_attn_int8(q_rot, t["k_cache"], t["v_cache"], t["k_scale"],
                                     t["v_scale"], t["seq_lens"], t["block_table"],
                                     max_seq_len=max_len, out=out, lse=lse, workspace=ws)
        else:
            kvd.rope_append_kv(t["q"], t["k_new"], t["v_new"], t["k_cache"], t["v_cache"],
                               t["positions"], t["block_table"], q_rot=q_rot)
            kvd.gqa_decode_attn(q_rot, t["k_cache"], t["v_cache"], t["seq_lens"],
                                t["block_table"], max_seq_len=max_len, out=out, lse=lse,
                                workspace=ws)
    return step


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("name,dtype", [("c2", "bf16"), ("c3", "bf16"), ("c3", "i8"),
                                        ("c4", "bf16")])
def test_graph_replays_equal_eager(name, dtype, fused):
    _graph_check(name, dtype, fused, 1)


@pytest.mark.parametrize("name", ["c3", "c4"])
def test_graph_replays_fused_multi_token(name):
    _graph_check(name, "bf16", True, 3)


def _graph_check(name, dtype, fused, T):
    dev = device()
    if name == "c2":
        s = W.spec("c2")
    elif name == "c3":
        s = W.spec("c3", batch=12, max_seq_len=2048, len_lo=1, len_hi=2048, q_gain=4.0)
    else:
        s = W.spec("c4", batch=6, num_blocks=1024, max_blocks_per_seq=128, len_lo=1,
                   len_hi=2048, q_gain=4.0)
    s = s.replace(dtype=dtype)
    p = W.make_problem(s) if T == 1 else W.make_window(s, T)
    print(f"[graph] {name} {dtype} fused={fused} T={T} B={s.batch} max_len={p.max_len}",
          flush=True)
    t = upload(p, dev)
    B, H, D = s.batch, s.n_heads, s.head_dim
    lead = (B,) if T == 1 else (B, T)
    q_rot = torch.empty((*lead, H, D), dtype=torch.float32, device=dev)
    out = torch.empty((*lead, H, D), dtype=torch.float32, device=dev)
    lse = torch.empty((*lead, H), dtype=torch.float32, device=dev)
    nbytes = kvd.workspace_size(q_rot, t["k_cache"], t["block_table"], p.max_len, n_query=T)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    step = _step_fn(t, s, p.max_len, (q_rot, out, lse, ws), fused=fused)
    step()
    torch.cuda.synchronize()
    ref = [x.clone() for x in (q_rot, out, lse, t["k_cache"], t["v_cache"])]

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    junk = torch.randn(1 << 20, device=dev)
    for rep in range(4):
        # the program's own work between replays: clobber the outputs
        for x in (q_rot, out, lse):
            x.fill_(float("nan"))
        junk.mul_(1.5)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = (q_rot, out, lse, t["k_cache"], t["v_cache"])
        for a, b in zip(got, ref):
            assert torch.equal(_bits(a), _bits(b)), f"replay {rep} differs"
    del graph
