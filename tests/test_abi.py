"""The C ABI without a GPU: the library loads, exports every function the
header declares, and rejects invalid arguments on the host before any HIP
call (nothing is enqueued, so these run on a machine with no GPU)."""
import ctypes
import os
import re

import pytest

from kv_cache_gqa_decode_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvdecode.h")

OK, EINVAL, EUNSUPPORTED, ERANGE, EWORKSPACE, EHIP = range(6)
FAKE = ctypes.c_void_p(0x1000)     # never dereferenced: validation fails first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) -
                  {"if", "sizeof", "defined"})


@pytest.fixture(scope="module")
def lib():
    return B.load_library()


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert set(names) == set(B.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n
    out = os.popen(f"nm -D --defined-only {B.LIB_PATH}").read()
    for n in names:
        assert re.search(rf"\bT {n}\b", out), f"{n} not exported"


def test_status_strings(lib):
    for code in range(6):
        assert lib.kvd_status_string(code)
    assert b"unknown" in lib.kvd_status_string(99)


def shape(**kw):
    base = dict(batch=2, n_heads=8, n_kv_heads=2, head_dim=64, kv_dtype=1, block_size=0,
                max_seq_len=64, num_blocks=0, max_blocks_per_seq=0)
    base.update(kw)
    return B.Shape(*base.values())


def attn(lib, sh, q=FAKE, k=FAKE, v=FAKE, lens=FAKE, table=None, msl=32, out=ctypes.c_void_p(0x2000),
         scale=0.125):
    return lib.gqa_decode_attn(ctypes.byref(sh) if sh is not None else None, q, k, v, lens, table,
                               msl, scale, out, None, None, 0, None)


def rope(lib, sh, q=FAKE, qr=ctypes.c_void_p(0x3000), table=None, base=10000.0, style=0):
    return lib.rope_append_kv(ctypes.byref(sh) if sh is not None else None, q, FAKE, FAKE, qr,
                              FAKE, FAKE, FAKE, table, base, style, None)


def test_attn_rejects_bad_arguments(lib):
    assert attn(lib, None) == EINVAL
    assert attn(lib, shape(n_heads=6, n_kv_heads=4)) == EINVAL          # H % G
    assert attn(lib, shape(head_dim=96)) == EUNSUPPORTED
    assert attn(lib, shape(head_dim=63)) == EUNSUPPORTED
    assert attn(lib, shape(kv_dtype=7)) == EUNSUPPORTED
    assert attn(lib, shape(block_size=64)) == EUNSUPPORTED
    assert attn(lib, shape(block_size=8)) == EUNSUPPORTED
    assert attn(lib, shape(block_size=32, max_seq_len=64, num_blocks=10,
                           max_blocks_per_seq=4), table=FAKE) == EINVAL  # 64 != 4 * 32
    assert attn(lib, shape(batch=-1)) == EINVAL
    assert attn(lib, shape(max_seq_len=0)) == EINVAL
    assert attn(lib, shape(), q=None) == EINVAL
    assert attn(lib, shape(), lens=None) == EINVAL
    assert attn(lib, shape(), out=None) == EINVAL
    assert attn(lib, shape(), out=FAKE) == EINVAL                        # out aliases q_rot
    assert attn(lib, shape(), k=ctypes.c_void_p(0x1004)) == EINVAL       # misaligned
    assert attn(lib, shape(), scale=float("nan")) == EINVAL
    assert attn(lib, shape(), msl=65) == ERANGE
    assert attn(lib, shape(), msl=-1) == ERANGE
    assert attn(lib, shape(), table=FAKE) == EINVAL                      # table for contiguous
    paged = shape(block_size=16, max_seq_len=64, num_blocks=10, max_blocks_per_seq=4)
    assert attn(lib, paged) == EINVAL                                    # missing table
    assert attn(lib, shape(block_size=16, max_seq_len=60, num_blocks=10,
                           max_blocks_per_seq=4), table=FAKE) == EINVAL  # 60 != 4 * 16
    assert attn(lib, shape(block_size=16, max_seq_len=64, num_blocks=0,
                           max_blocks_per_seq=4), table=FAKE) == EINVAL
    assert attn(lib, shape(batch=0)) == OK                               # nothing to do


def step(lib, sh, q=FAKE, k=FAKE, pos=FAKE, table=None, msl=32, out=ctypes.c_void_p(0x2000),
         qr=None, base=10000.0, style=0, scale=0.125, opts=None, kn=FAKE):
    return lib.gqa_decode_step(ctypes.byref(sh) if sh is not None else None, q, kn, FAKE, k, k,
                               pos, table, msl, base, style, scale, qr, out, None, None, 0, opts,
                               None)


def test_step_rejects_bad_arguments(lib):
    assert step(lib, None) == EINVAL
    assert step(lib, shape(kv_dtype=2)) == EUNSUPPORTED                 # INT8: its own call
    assert step(lib, shape(kv_dtype=0)) == EUNSUPPORTED                 # fp32: two calls
    assert step(lib, shape(n_heads=128, n_kv_heads=2)) == EUNSUPPORTED  # 64 heads per KV head
    assert step(lib, shape(head_dim=96)) == EUNSUPPORTED
    assert step(lib, shape(), style=2) == EUNSUPPORTED
    assert step(lib, shape(), q=None) == EINVAL
    assert step(lib, shape(), pos=None) == EINVAL
    assert step(lib, shape(), out=None) == EINVAL
    assert step(lib, shape(), out=FAKE) == EINVAL                       # out aliases q
    assert step(lib, shape(), qr=ctypes.c_void_p(0x2000)) == EINVAL     # q_rot aliases out
    assert step(lib, shape(), q=ctypes.c_void_p(0x1008)) == EINVAL      # misaligned
    assert step(lib, shape(), kn=ctypes.c_void_p(0x1008)) == EINVAL     # k_new misaligned
    assert step(lib, shape(), base=0.0) == EINVAL
    assert step(lib, shape(), scale=float("inf")) == EINVAL
    assert step(lib, shape(), table=FAKE) == EINVAL                     # table for contiguous
    assert step(lib, shape(), msl=0) == ERANGE                          # the step attends a token
    assert step(lib, shape(), msl=65) == ERANGE
    vopt = B._COptions(1, 0, 0, 0, 0, 0, None, None)                     # VALU kernel asked for
    assert step(lib, shape(), opts=ctypes.byref(vopt)) == EINVAL
    assert step(lib, shape(batch=0)) == OK                              # nothing to do


def step8(lib, sh, ks=FAKE, vs=FAKE, msl=32):
    return lib.gqa_decode_step_int8(ctypes.byref(sh) if sh is not None else None, FAKE, FAKE,
                                    FAKE, FAKE, FAKE, ks, vs, FAKE, None, msl, 10000.0, 0, 0.125,
                                    None, ctypes.c_void_p(0x2000), None, None, 0, None, None)


def test_step_int8_validates(lib):
    assert step8(lib, None) == EINVAL
    assert step8(lib, shape()) == EUNSUPPORTED                          # a bf16 shape
    assert step8(lib, shape(kv_dtype=2), ks=None) == EINVAL             # scales missing
    assert step8(lib, shape(kv_dtype=2, n_heads=64, n_kv_heads=2)) == EUNSUPPORTED
    assert step8(lib, shape(kv_dtype=2), msl=0) == ERANGE
    assert step8(lib, shape(kv_dtype=2, batch=0)) == OK


def stepm(lib, sh, T, msl=32):
    return lib.gqa_decode_step_multi(ctypes.byref(sh) if sh is not None else None, T, FAKE, FAKE,
                                     FAKE, FAKE, FAKE, FAKE, None, msl, 10000.0, 0, 0.125, None,
                                     ctypes.c_void_p(0x2000), None, None, 0, None, None)


def test_step_multi_validates(lib):
    assert stepm(lib, None, 2) == EINVAL
    for T in (0, -1, 17):                                               # 1 to 16 new tokens
        assert stepm(lib, shape(), T) == EUNSUPPORTED
    assert stepm(lib, shape(n_heads=8, n_kv_heads=2), 9) == EUNSUPPORTED   # 36 rows per KV head
    assert stepm(lib, shape(kv_dtype=2), 2) == EUNSUPPORTED             # bf16 caches only
    assert stepm(lib, shape(), 2, msl=0) == ERANGE
    assert stepm(lib, shape(batch=0, n_heads=2, n_kv_heads=2), 16) == OK


def test_rope_rejects_bad_arguments(lib):
    assert rope(lib, None) == EINVAL
    assert rope(lib, shape(head_dim=80)) == EUNSUPPORTED
    assert rope(lib, shape(), style=2) == EUNSUPPORTED
    assert rope(lib, shape(), qr=None) == EINVAL
    assert rope(lib, shape(), qr=FAKE) == EINVAL                         # q_rot aliases q
    assert rope(lib, shape(), base=0.0) == EINVAL
    assert rope(lib, shape(), base=float("inf")) == EINVAL
    assert rope(lib, shape(), table=FAKE) == EINVAL
    assert rope(lib, shape(block_size=16, max_seq_len=64, num_blocks=4,
                           max_blocks_per_seq=4)) == EINVAL
    assert rope(lib, shape(batch=0)) == OK


def rope8(lib, sh, ks=FAKE, vs=FAKE, table=None):
    return lib.rope_append_kv_int8(ctypes.byref(sh) if sh is not None else None, FAKE, FAKE,
                                   FAKE, ctypes.c_void_p(0x3000), FAKE, FAKE, ks, vs, FAKE, table,
                                   10000.0, 0, None)


def attn8(lib, sh, ks=FAKE, vs=FAKE, msl=32):
    return lib.gqa_decode_attn_int8(ctypes.byref(sh) if sh is not None else None, FAKE, FAKE,
                                    FAKE, ks, vs, FAKE, None, msl, 0.125,
                                    ctypes.c_void_p(0x2000), None, None, 0, None)


def test_int8_calls_validate(lib):
    i8 = shape(kv_dtype=2)
    # the bf16/fp32 calls reject INT8 caches (they carry no scales) and the
    # INT8 calls reject the other dtypes
    assert rope(lib, i8) == EUNSUPPORTED
    assert attn(lib, i8) == EUNSUPPORTED
    assert rope8(lib, shape()) == EUNSUPPORTED
    assert attn8(lib, shape()) == EUNSUPPORTED
    assert rope8(lib, None) == EINVAL and attn8(lib, None) == EINVAL
    assert rope8(lib, i8, ks=None) == EINVAL and rope8(lib, i8, vs=None) == EINVAL
    assert attn8(lib, i8, ks=None) == EINVAL and attn8(lib, i8, vs=None) == EINVAL
    # contiguous INT8 capacity must be whole 16-token groups
    assert rope8(lib, shape(kv_dtype=2, max_seq_len=40)) == EUNSUPPORTED
    assert attn8(lib, shape(kv_dtype=2, max_seq_len=40)) == EUNSUPPORTED
    assert attn8(lib, i8, msl=65) == ERANGE
    assert rope8(lib, i8, table=FAKE) == EINVAL
    assert rope8(lib, shape(kv_dtype=2, batch=0)) == OK
    assert attn8(lib, shape(kv_dtype=2, batch=0)) == OK


def rope_m(lib, sh, T, ks=None, vs=None):
    return lib.rope_append_kv_multi(ctypes.byref(sh) if sh is not None else None, T, FAKE, FAKE,
                                    FAKE, ctypes.c_void_p(0x3000), FAKE, FAKE, ks, vs, FAKE, None,
                                    10000.0, 0, None)


def attn_m(lib, sh, T, ks=None, vs=None, msl=32, opts=None, scale=0.125):
    return lib.gqa_decode_attn_multi(ctypes.byref(sh) if sh is not None else None, T, FAKE, FAKE,
                                     FAKE, ks, vs, FAKE, None, msl, scale,
                                     ctypes.c_void_p(0x2000), None, None, 0,
                                     None if opts is None else ctypes.byref(opts), None)


def test_multi_calls_validate(lib):
    bf, i8 = shape(), shape(kv_dtype=2)
    assert rope_m(lib, None, 2) == EINVAL and attn_m(lib, None, 2) == EINVAL
    for T in (0, -1, 65):                # the window must fit the cache (64 slots)
        assert rope_m(lib, bf, T) == EUNSUPPORTED
    for T in (0, -1, 33):                # the decode kernels take up to 32 query rows
        assert attn_m(lib, bf, T) == EUNSUPPORTED
    # scales exactly for INT8 caches
    assert rope_m(lib, bf, 2, ks=FAKE, vs=FAKE) == EINVAL
    assert attn_m(lib, bf, 2, ks=FAKE) == EINVAL
    assert rope_m(lib, i8, 2) == EINVAL and attn_m(lib, i8, 2, ks=FAKE) == EINVAL
    assert attn_m(lib, bf, 2, msl=65) == ERANGE
    assert rope_m(lib, shape(batch=0), 5) == OK
    assert attn_m(lib, shape(batch=0), 5) == OK
    assert attn_m(lib, shape(kv_dtype=2, batch=0), 5, ks=FAKE, vs=FAKE) == OK
    assert lib.gqa_decode_workspace_size_multi(ctypes.byref(bf), 0, 10, None) == 0


def prefill(lib, sh, T, q=FAKE, lens=FAKE, table=None, msl=32, out=ctypes.c_void_p(0x2000),
            opts=None, ws=None, ws_bytes=0):
    return lib.gqa_prefill_attn(ctypes.byref(sh) if sh is not None else None, T, q, FAKE, FAKE,
                                lens, table, msl, 0.125, out, None, ws, ws_bytes,
                                None if opts is None else ctypes.byref(opts), None)


def test_prefill_validates(lib):
    assert prefill(lib, None, 4) == EINVAL
    assert prefill(lib, shape(kv_dtype=0), 4) == EUNSUPPORTED          # fp32 cache
    assert prefill(lib, shape(kv_dtype=2), 4) == EUNSUPPORTED          # INT8 cache
    for T in (0, -3, 65):
        assert prefill(lib, shape(), T) == EUNSUPPORTED
    assert prefill(lib, shape(), 4, q=None) == EINVAL
    assert prefill(lib, shape(), 4, lens=None) == EINVAL
    assert prefill(lib, shape(), 4, out=FAKE) == EINVAL                # out aliases q_rot
    assert prefill(lib, shape(), 4, table=FAKE) == EINVAL
    assert prefill(lib, shape(), 4, msl=65) == ERANGE
    assert prefill(lib, shape(batch=0), 64) == OK
    # options: key splits of whole 32-token tiles, a prefill dispatch order
    # (6-8) and timing events (both or neither); no kernel or tail fields,
    # no decode order
    assert prefill(lib, shape(batch=0), 4, opts=B._COptions()) == OK
    assert prefill(lib, shape(batch=0), 4, opts=B._COptions(split_tokens=64)) == OK
    assert prefill(lib, shape(batch=0), 4, opts=B._COptions(split_tokens=16)) == EINVAL
    assert prefill(lib, shape(batch=0), 4, opts=B._COptions(split_tokens=-32)) == EINVAL
    assert prefill(lib, shape(batch=0), 4, opts=B._COptions(tail_split_tokens=32)) == EINVAL
    assert prefill(lib, shape(batch=0), 4, opts=B._COptions(kernel=2)) == EINVAL
    assert prefill(lib, shape(batch=0), 4, opts=B._COptions(event_start=0x10)) == EINVAL
    for order in (6, 7, 8):
        assert prefill(lib, shape(batch=0), 4, opts=B._COptions(dispatch_order=order)) == OK
    for order in (1, 2, 3, 4, 5, 9, -1):
        assert prefill(lib, shape(batch=0), 4, opts=B._COptions(dispatch_order=order)) == EINVAL


def test_prefill_int8_validates(lib):
    """The INT8 prefill takes INT8 shapes and both scales; the bf16 one
    refuses INT8 shapes; the workspace size serves both."""
    O = B._COptions

    def pf8(sh, ks=FAKE, vs=FAKE, opts=None, msl=32):
        return lib.gqa_prefill_attn_int8(ctypes.byref(sh), 4, FAKE, FAKE, FAKE, ks, vs, FAKE,
                                         None, msl, 0.0, ctypes.c_void_p(0x2000), None, None, 0,
                                         None if opts is None else ctypes.byref(opts), None)

    i8 = shape(kv_dtype=2)
    assert pf8(shape()) == EUNSUPPORTED                         # bf16 shape
    assert pf8(i8, ks=None) == EINVAL and pf8(i8, vs=None) == EINVAL
    assert pf8(shape(kv_dtype=2, batch=0)) == OK
    assert pf8(i8, opts=O(kernel=3)) == EINVAL
    assert pf8(i8, opts=O(split_tokens=16)) == EINVAL          # whole 32-token tiles
    assert pf8(i8, opts=O(split_tokens=32), msl=64) == EWORKSPACE   # two splits, no workspace
    assert prefill(lib, i8, 4) == EUNSUPPORTED
    sh = shape(kv_dtype=2, max_seq_len=256)
    n = lib.gqa_prefill_workspace_size(ctypes.byref(sh), 4, 256, ctypes.byref(O(split_tokens=64)))
    assert n == lib.gqa_prefill_workspace_size(ctypes.byref(shape(max_seq_len=256)), 4, 256,
                                               ctypes.byref(O(split_tokens=64))) > 0


def test_prefill_key_split_workspace(lib):
    """A requested key split sizes its partials, (o[D], log2 lse) per query
    row and split, each array 256-byte aligned; without that workspace the
    call is refused before anything is enqueued."""
    O = B._COptions
    sh = shape(batch=2, n_heads=8, n_kv_heads=2, head_dim=64, max_seq_len=256)
    T = 4
    rows = 2 * T * 8
    up = lambda x: (x + 255) // 256 * 256
    for split, msl, n in ((64, 256, 4), (96, 256, 3), (32, 33, 2)):
        size = lib.gqa_prefill_workspace_size(ctypes.byref(sh), T, msl,
                                              ctypes.byref(O(split_tokens=split)))
        assert size == up(rows * n * 64 * 4) + up(rows * n * 4), (split, msl)
        assert prefill(lib, sh, T, msl=msl, opts=O(split_tokens=split)) == EWORKSPACE
        assert prefill(lib, sh, T, msl=msl, opts=O(split_tokens=split), ws=FAKE,
                       ws_bytes=size - 1) == EWORKSPACE
        assert prefill(lib, sh, T, msl=msl, opts=O(split_tokens=split),
                       ws=ctypes.c_void_p(0x1010), ws_bytes=size) == EWORKSPACE   # misaligned
    # one split covers the window: no workspace
    assert lib.gqa_prefill_workspace_size(ctypes.byref(sh), T, 64,
                                          ctypes.byref(O(split_tokens=64))) == 0
    # invalid arguments report 0
    assert lib.gqa_prefill_workspace_size(ctypes.byref(sh), T, 64,
                                          ctypes.byref(O(split_tokens=48))) == 0
    assert lib.gqa_prefill_workspace_size(ctypes.byref(sh), T, 257, None) == 0
    assert lib.gqa_prefill_workspace_size(None, T, 64, None) == 0


def test_mixed_validates(lib):
    """Mixed-precision calls: an INT8 history, a window in [1, max_seq_len],
    both rings; no kernel or tail options; batch 0 does nothing."""
    O = B._COptions
    i8 = shape(kv_dtype=2)

    def app(sh, window, kr=FAKE, vr=FAKE, ks=FAKE):
        return lib.rope_append_kv_mixed(ctypes.byref(sh), window, FAKE, FAKE, FAKE,
                                        ctypes.c_void_p(0x3000), FAKE, FAKE, ks, FAKE, kr, vr,
                                        FAKE, None, 10000.0, 0, None)

    def att(sh, window, kr=FAKE, opts=None, msl=32, ws=None, ws_bytes=0):
        return lib.gqa_decode_attn_mixed(ctypes.byref(sh), window, FAKE, FAKE, FAKE, FAKE, FAKE,
                                         kr, FAKE, FAKE, None, msl, 0.0, ctypes.c_void_p(0x2000),
                                         None, ws, ws_bytes,
                                         None if opts is None else ctypes.byref(opts), None)

    assert app(shape(), 16) == EUNSUPPORTED                 # bf16 shape
    assert app(i8, 0) == ERANGE and app(i8, 65) == ERANGE
    assert app(i8, 16, kr=None) == EINVAL and app(i8, 16, ks=None) == EINVAL
    assert app(shape(kv_dtype=2, batch=0), 16) == OK
    assert att(shape(), 16) == EUNSUPPORTED
    assert att(i8, 0) == ERANGE and att(i8, 65) == ERANGE
    assert att(i8, 16, kr=None) == EINVAL
    assert att(i8, 16, msl=65) == ERANGE
    for bad in (O(kernel=2), O(tail_split_tokens=32), O(dispatch_order=7)):
        assert att(i8, 16, opts=bad) == EINVAL
    empty = shape(kv_dtype=2, batch=0)
    assert att(empty, 16) == OK and att(empty, 16, opts=O(split_tokens=64)) == OK
    assert lib.gqa_decode_workspace_size_mixed(ctypes.byref(empty), 16, 32, None) == 0
    assert lib.gqa_decode_workspace_size_mixed(ctypes.byref(i8), 0, 32, None) == 0
    assert lib.gqa_decode_workspace_size_mixed(ctypes.byref(shape()), 16, 32, None) == 0


def test_options_validation(lib):
    """kvd_options travel with the call; bad values are refused before any
    HIP call (batch 0: a valid call does nothing)."""
    O = B._COptions
    empty = shape(batch=0)
    assert attn_m(lib, empty, 1, opts=O()) == OK                       # zeros: automatic
    for bad in (O(kernel=-1), O(kernel=4), O(split_tokens=24), O(split_tokens=-16),
                O(split_tokens=8192 + 16), O(tail_split_tokens=8), O(tail_span_tokens=-1),
                O(dispatch_order=-1), O(dispatch_order=6), O(dispatch_order=8),
                O(dispatch_order=9), O(reserved=1),
                O(event_start=0x10), O(event_stop=0x10)):
        assert attn_m(lib, empty, 1, opts=bad) == EINVAL
        assert lib.gqa_decode_workspace_size_multi(ctypes.byref(shape()), 1, 32,
                                                   ctypes.byref(bad)) == 0
    for good in (O(kernel=1), O(kernel=2, split_tokens=8192), O(split_tokens=16),
                 O(dispatch_order=5), O(tail_split_tokens=32, tail_span_tokens=64)):
        assert attn_m(lib, empty, 1, opts=good) == OK
    plan = (ctypes.c_int32 * 4)()
    assert lib.kvd_get_plan_multi(ctypes.byref(shape()), 1, 32, ctypes.byref(O(kernel=9)),
                                  plan) == EINVAL


def test_scale_zero_selects_the_default(lib):
    """0 asks the library for 1/sqrt(head_dim); infinities and NaN are refused."""
    empty = shape(batch=0)
    assert attn_m(lib, empty, 1, scale=0.0) == OK
    assert attn(lib, empty, scale=0.0) == OK
    assert attn_m(lib, shape(), 1, scale=float("inf")) == EINVAL
    assert attn_m(lib, shape(), 1, scale=float("-inf")) == EINVAL


def test_plan_validation(lib):
    plan = (ctypes.c_int32 * 4)()
    assert lib.kvd_get_plan(None, 0, plan) == EINVAL
    assert lib.kvd_get_plan(ctypes.byref(shape()), 100, plan) == ERANGE
    assert lib.gqa_decode_workspace_size(ctypes.byref(shape(head_dim=48)), 10) == 0


def test_binding_raises_without_compute(lib):
    import torch
    cpu = torch.zeros((2, 8, 64), dtype=torch.float32)
    with pytest.raises(ValueError):
        B._dtype_code(torch.float16)
    with pytest.raises(ValueError):
        B.make_shape(2, 8, torch.zeros((2, 64, 2)), None)
    with pytest.raises(ValueError):
        B._options(B.Options(kernel="triton"))
    with pytest.raises(ValueError):
        B._scale_arg(0.0)
    assert B._scale_arg(None) == 0.0
    assert cpu.shape == (2, 8, 64)


def test_read_probe_validates(lib):
    sink = ctypes.c_void_p(0x2000)
    assert lib.kvd_read_probe(FAKE, 4096, sink, 4, 8, 8, None) == EINVAL        # unknown mode bit
    assert lib.kvd_read_probe(FAKE, 4096 + 16, sink, 4, 8, 4, None) == EINVAL   # LDS: whole KiB
    assert lib.kvd_read_probe(FAKE, 4100, sink, 4, 8, 0, None) == EINVAL        # 16-byte words
    assert lib.kvd_read_probe(FAKE, 4096, sink, 4, 3, 0, None) == EUNSUPPORTED  # unroll
    assert lib.kvd_read_probe(ctypes.c_void_p(0x1008), 4096, sink, 4, 8, 0, None) == EINVAL
    assert lib.kvd_read_probe(FAKE, 4096, sink, 0, 8, 0, None) == EINVAL
