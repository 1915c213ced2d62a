"""The streaming-read probe (the measured read ceiling the benchmark reports
beside the nominal peak) reads every byte: on the register path the XOR of
the per-workgroup words equals the XOR of the whole buffer; the HBM -> LDS
path runs over the same buffer in every launch shape the benchmark sweeps."""
import numpy as np
import pytest
import torch

import kv_cache_gqa_decode_amd as kvd
from kv_cache_gqa_decode_amd import _binding as B
from tests.gpu_helpers import device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("mode", [0, B.PROBE_CHUNKED, B.PROBE_NONTEMPORAL,
                                  B.PROBE_CHUNKED | B.PROBE_NONTEMPORAL])
@pytest.mark.parametrize("unroll", [1, 4, 16])
def test_register_probe_reads_every_word(mode, unroll):
    dev = device()
    rng = np.random.default_rng(5)
    host = rng.integers(0, 2 ** 32, size=(3 << 18) + 4 * 37, dtype=np.uint32)  # ragged tail
    buf = torch.from_numpy(host.view(np.int32)).to(dev)
    for nwg in (1, 7, 256):
        sink = kvd.read_probe(buf, nwg, unroll, mode)
        torch.cuda.synchronize()
        got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
        assert got == np.bitwise_xor.reduce(host), f"mode {mode} unroll {unroll} nwg {nwg}"


@pytest.mark.parametrize("mode", [B.PROBE_LDS, B.PROBE_LDS | B.PROBE_NONTEMPORAL])
@pytest.mark.parametrize("unroll", [1, 4, 8, 16])
def test_lds_probe_runs(mode, unroll):
    dev = device()
    buf = torch.arange(1 << 20, dtype=torch.int32, device=dev)     # 4 MiB, whole KiB pieces
    for nwg in (1, 5, 256, 2048):
        sink = kvd.read_probe(buf, nwg, unroll, mode)
        torch.cuda.synchronize()
        assert sink.numel() == nwg
