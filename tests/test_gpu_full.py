"""GPU parity at the full workload sizes, in the launch configuration the
benchmark uses (automatic plan).

Every (b, h) output row and its lse are compared with the oracle, which
computes the whole batch (fp64, all host threads); every appended cache row
is compared bit for bit, and the rest of each cache is checked unchanged on
the device against the host copy.
"""
import numpy as np
import pytest
import torch

from kv_cache_gqa_decode_amd import workloads as W
from tests import gates
from tests.gpu_helpers import (appended_rows, assert_q_rot, bits, device, gpu_step, oracle_step,
                               upload)

pytestmark = pytest.mark.gpu


def run_full(s: W.Spec):
    dev = device()
    p = W.make_problem(s)
    print(f"[full] {s.name} G={s.n_kv_heads} B={s.batch} max_len={p.max_len}", flush=True)
    t = upload(p, dev)
    q_rot, out, lse = gpu_step(t, s, p.max_len)
    oq, oo, ol, okc, ovc = oracle_step(p)
    assert_q_rot(q_rot.cpu().numpy(), oq, f"{s.name} q_rot")
    e = gates.assert_out(out.cpu().numpy(), oo, s.dtype, f"{s.name} all rows")
    gates.assert_lse(lse.cpu().numpy(), ol, s.dtype, f"{s.name} all rows lse")
    print(f"[full] {s.name} G={s.n_kv_heads}: {e}", flush=True)
    # appended rows, bit for bit
    kc = t["k_cache"]
    vc = t["v_cache"]
    for (i0, i1) in appended_rows(p):
        assert np.array_equal(bits(W.from_torch(kc[i0, i1])), bits(okc[i0, i1]))
        assert np.array_equal(bits(W.from_torch(vc[i0, i1])), bits(ovc[i0, i1]))
    # nothing else moved: compare the whole caches on the device
    ek = W.as_torch(okc, dev)
    assert torch.equal(kc.view(torch.int16), ek.view(torch.int16))
    del ek
    ev = W.as_torch(ovc, dev)
    assert torch.equal(vc.view(torch.int16), ev.view(torch.int16))
    del ev, t
    torch.cuda.empty_cache()


def test_c3_batched_varlen_full():
    run_full(W.spec("c3"))


def test_c4_paged_full():
    run_full(W.spec("c4"))


@pytest.mark.parametrize("G", [32, 8, 1])
def test_c5_long_context_full(G):
    run_full(W.spec("c5", n_kv_heads=G))


@pytest.mark.parametrize("G", [8, 1])
def test_c5_peaked(G):
    """q x 32: score spread ~2.8, so the running max moves and rescales."""
    run_full(W.spec("c5", n_kv_heads=G, q_gain=32.0))
