"""ctypes binding of libkvdecode.so (argument marshalling only).

Every step of the decode computation runs in the HIP kernels behind the C
ABI (include/kvdecode.h).  This module checks tensor devices, dtypes and
shapes, allocates outputs and the split workspace with torch, passes raw
pointers and the current HIP stream, and turns status codes into
exceptions.  There is no fallback: without the built library every call
raises.

The split workspace, when the caller passes none, is allocated per call
through torch's caching allocator on the call's stream: calls on different
streams never share one, and under graph capture the graph's memory pool
keeps it alive for the graph's lifetime.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import threading
from typing import Optional, Tuple

import torch

# KVD_LIBRARY_PATH may point at another build of the same library (for A/B
# measurements of build variants); by default the in-tree build is used.
LIB_PATH = os.environ.get("KVD_LIBRARY_PATH") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libkvdecode.so")

KVD_FP32, KVD_BF16, KVD_INT8 = 0, 1, 2
_STYLES = {"interleaved": 0, "half": 1}
# kvd_kernel values
_KERNELS = {None: 0, "auto": 0, "valu": 1, "mfma": 2, "int8": 3}
_KERNEL_NAMES = {1: "valu", 2: "mfma", 3: "int8"}


class KvdError(ValueError):
    """A non-OK status from libkvdecode.so."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "n_heads", "n_kv_heads", "head_dim", "kv_dtype", "block_size",
        "max_seq_len", "num_blocks", "max_blocks_per_seq")]


class _COptions(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int32), ("split_tokens", ctypes.c_int32),
                ("tail_split_tokens", ctypes.c_int32), ("tail_span_tokens", ctypes.c_int32),
                ("dispatch_order", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("event_start", ctypes.c_void_p), ("event_stop", ctypes.c_void_p)]


# prefill dispatch orders (Options.dispatch_order of gqa_prefill_attn)
PREFILL_PAIRS_FASTEST, PREFILL_TILES_FASTEST, PREFILL_XCD_RUNS = 5, 6, 7


@dataclasses.dataclass(frozen=True)
class Options:
    """Per-call plan overrides and timing events (kvd_options).

    kernel          None / "auto", "valu", "mfma" or "int8"
    split_tokens    tokens per split (0 automatic; a multiple of 16 up to 8192)
    tail_split_tokens, tail_span_tokens
                    shorter splits over the last positions (0: none / automatic)
    dispatch_order  None (automatic), a decode unit order 0-4: 0 split
                    fastest, 1 head-sequence-split, 2 head-split-sequence,
                    3 device-built work list, 4 work list derived in the split
                    kernel; or a prefill order: PREFILL_PAIRS_FASTEST,
                    PREFILL_TILES_FASTEST, PREFILL_XCD_RUNS
    events          None, or (start, stop) torch.cuda.Event(enable_timing=True)
                    recorded on the call's stream around its main kernel
    """
    kernel: Optional[str] = None
    split_tokens: int = 0
    tail_split_tokens: int = 0
    tail_span_tokens: int = 0
    dispatch_order: Optional[int] = None
    events: Optional[Tuple[object, object]] = None

    def with_events(self, start, stop) -> "Options":
        return dataclasses.replace(self, events=(start, stop))


def _event_handle(ev) -> int:
    """The hipEvent_t behind a torch.cuda.Event (torch creates it lazily on
    its first record)."""
    h = ev.cuda_event
    if not h:
        ev.record()
        h = ev.cuda_event
    return h


def _options(opts: Optional[Options]):
    if opts is None:
        return None
    if opts.kernel not in _KERNELS:
        raise ValueError(f"kernel must be one of {sorted(k for k in _KERNELS if k)}")
    c = _COptions(_KERNELS[opts.kernel], int(opts.split_tokens), int(opts.tail_split_tokens),
                  int(opts.tail_span_tokens),
                  0 if opts.dispatch_order is None else int(opts.dispatch_order) + 1, 0, None, None)
    if opts.events is not None:
        c.event_start = _event_handle(opts.events[0])
        c.event_stop = _event_handle(opts.events[1])
    return ctypes.byref(c)


EXPORTED = ("rope_append_kv", "gqa_decode_attn", "rope_append_kv_int8",
            "gqa_decode_attn_int8", "gqa_decode_workspace_size", "rope_append_kv_multi",
            "gqa_decode_attn_multi", "gqa_decode_workspace_size_multi", "gqa_prefill_attn",
            "gqa_prefill_workspace_size", "gqa_prefill_attn_int8", "rope_append_kv_mixed",
            "gqa_decode_attn_mixed",
            "gqa_decode_workspace_size_mixed",
            "kvd_status_string", "kvd_get_plan", "kvd_get_plan_multi", "kvd_read_probe",
            "gqa_decode_attn_multi_noalloc", "gqa_decode_step", "gqa_decode_step_int8",
            "gqa_decode_step_multi")
NOALLOC_SCRATCH_BYTES = 32 << 20     # KVD_NOALLOC_SCRATCH_BYTES

_lib = None
_lock = threading.Lock()


def library_path() -> str:
    return LIB_PATH


def load_library():
    """Load libkvdecode.so once; raise if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m "
                "kv_cache_gqa_decode_amd.build` (or __graft_entry__.build())")
        lib = ctypes.CDLL(LIB_PATH)
        P, I32 = ctypes.c_void_p, ctypes.c_int32
        SP = ctypes.POINTER(Shape)
        lib.rope_append_kv.restype = I32
        lib.rope_append_kv.argtypes = [SP, P, P, P, P, P, P, P, P, ctypes.c_double, I32, P]
        lib.gqa_decode_attn.restype = I32
        lib.gqa_decode_attn.argtypes = [SP, P, P, P, P, P, I32, ctypes.c_float, P, P, P,
                                        ctypes.c_size_t, P]
        lib.rope_append_kv_int8.restype = I32
        lib.rope_append_kv_int8.argtypes = [SP, P, P, P, P, P, P, P, P, P, P,
                                            ctypes.c_double, I32, P]
        lib.gqa_decode_attn_int8.restype = I32
        lib.gqa_decode_attn_int8.argtypes = [SP, P, P, P, P, P, P, P, I32, ctypes.c_float, P,
                                             P, P, ctypes.c_size_t, P]
        lib.gqa_decode_workspace_size.restype = ctypes.c_size_t
        lib.gqa_decode_workspace_size.argtypes = [SP, I32]
        lib.rope_append_kv_multi.restype = I32
        lib.rope_append_kv_multi.argtypes = [SP, I32, P, P, P, P, P, P, P, P, P, P,
                                             ctypes.c_double, I32, P]
        lib.gqa_decode_attn_multi.restype = I32
        OP = ctypes.POINTER(_COptions)
        lib.gqa_decode_attn_multi.argtypes = [SP, I32, P, P, P, P, P, P, P, I32, ctypes.c_float,
                                              P, P, P, ctypes.c_size_t, OP, P]
        lib.gqa_decode_attn_multi_noalloc.restype = I32
        lib.gqa_decode_attn_multi_noalloc.argtypes = [SP, I32, P, P, P, P, P, P, P, I32,
                                                      ctypes.c_float, P, P, OP, P]
        lib.gqa_prefill_attn.restype = I32
        lib.gqa_prefill_attn.argtypes = [SP, I32, P, P, P, P, P, I32, ctypes.c_float, P, P, P,
                                         ctypes.c_size_t, OP, P]
        lib.gqa_prefill_attn_int8.restype = I32
        lib.gqa_prefill_attn_int8.argtypes = [SP, I32, P, P, P, P, P, P, P, I32, ctypes.c_float,
                                              P, P, P, ctypes.c_size_t, OP, P]
        lib.gqa_prefill_workspace_size.restype = ctypes.c_size_t
        lib.gqa_prefill_workspace_size.argtypes = [SP, I32, I32, OP]
        lib.rope_append_kv_mixed.restype = I32
        lib.rope_append_kv_mixed.argtypes = [SP, I32, P, P, P, P, P, P, P, P, P, P, P, P,
                                             ctypes.c_double, I32, P]
        lib.gqa_decode_attn_mixed.restype = I32
        lib.gqa_decode_attn_mixed.argtypes = [SP, I32, P, P, P, P, P, P, P, P, P, I32,
                                              ctypes.c_float, P, P, P, ctypes.c_size_t, OP, P]
        lib.gqa_decode_workspace_size_mixed.restype = ctypes.c_size_t
        lib.gqa_decode_workspace_size_mixed.argtypes = [SP, I32, I32, OP]
        lib.gqa_decode_step_int8.restype = I32
        lib.gqa_decode_step_int8.argtypes = [SP, P, P, P, P, P, P, P, P, P, I32, ctypes.c_double,
                                             I32, ctypes.c_float, P, P, P, P, ctypes.c_size_t, OP,
                                             P]
        lib.gqa_decode_step.restype = I32
        lib.gqa_decode_step.argtypes = [SP, P, P, P, P, P, P, P, I32, ctypes.c_double, I32,
                                        ctypes.c_float, P, P, P, P, ctypes.c_size_t, OP, P]
        lib.gqa_decode_step_multi.restype = I32
        lib.gqa_decode_step_multi.argtypes = [SP, I32, P, P, P, P, P, P, P, I32, ctypes.c_double,
                                              I32, ctypes.c_float, P, P, P, P, ctypes.c_size_t,
                                              OP, P]
        lib.gqa_decode_workspace_size_multi.restype = ctypes.c_size_t
        lib.gqa_decode_workspace_size_multi.argtypes = [SP, I32, I32, OP]
        lib.kvd_status_string.restype = ctypes.c_char_p
        lib.kvd_status_string.argtypes = [I32]
        lib.kvd_get_plan.restype = I32
        lib.kvd_get_plan.argtypes = [SP, I32, ctypes.POINTER(I32)]
        lib.kvd_get_plan_multi.restype = I32
        lib.kvd_get_plan_multi.argtypes = [SP, I32, I32, OP, ctypes.POINTER(I32)]
        lib.kvd_read_probe.restype = I32
        lib.kvd_read_probe.argtypes = [P, ctypes.c_size_t, P, I32, I32, I32, P]
        _lib = lib
        return lib


def _check(status: int) -> None:
    if status != 0:
        msg = load_library().kvd_status_string(status).decode()
        raise KvdError(status, msg)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return KVD_FP32
    if dt == torch.bfloat16:
        return KVD_BF16
    if dt == torch.int8:
        return KVD_INT8
    raise ValueError(f"unsupported KV dtype {dt}: float32, bfloat16 or int8")


def _need(t: torch.Tensor, name: str, device: torch.device, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def make_shape(batch: int, n_heads: int, k_cache: torch.Tensor,
               block_table: Optional[torch.Tensor]) -> Shape:
    """kvd_shape from the K cache tensor: contiguous [B, S_max, G, D] or paged
    pool [num_blocks, 16, G, D] with table [B, max_blocks_per_seq]; an int8
    K cache is grouped by 16 tokens: [B, S_max/16, G, 16, D] or
    [num_blocks, G, 16, D]."""
    if k_cache.dtype == torch.int8:
        if block_table is None:
            if k_cache.dim() != 5 or int(k_cache.shape[3]) != 16:
                raise ValueError("contiguous int8 K cache must be [B, S_max/16, G, 16, D]")
            if int(k_cache.shape[0]) != batch:
                raise ValueError("contiguous cache batch dimension does not match q")
            return Shape(batch, n_heads, int(k_cache.shape[2]), int(k_cache.shape[4]), KVD_INT8,
                         0, int(k_cache.shape[1]) * 16, 0, 0)
        # paged: [NB, G, 16, D] (16-token blocks) or [NB, m, G, 16, D] (16m-token blocks)
        if k_cache.dim() == 4 and int(k_cache.shape[2]) == 16:
            nb, m, G, D = int(k_cache.shape[0]), 1, int(k_cache.shape[1]), int(k_cache.shape[3])
        elif k_cache.dim() == 5 and int(k_cache.shape[3]) == 16:
            nb, m, G, D = (int(k_cache.shape[i]) for i in (0, 1, 2, 4))
        else:
            raise ValueError("paged int8 K pool must be [num_blocks, G, 16, D] or "
                             "[num_blocks, block_size/16, G, 16, D]")
        if block_table.dim() != 2 or int(block_table.shape[0]) != batch:
            raise ValueError("block_table must be [batch, max_blocks_per_seq]")
        mbps = int(block_table.shape[1])
        return Shape(batch, n_heads, G, D, KVD_INT8, 16 * m, mbps * 16 * m, nb, mbps)
    if k_cache.dim() != 4:
        raise ValueError("cache must be 4-D")
    G, D = int(k_cache.shape[2]), int(k_cache.shape[3])
    code = _dtype_code(k_cache.dtype)
    if block_table is None:
        if int(k_cache.shape[0]) != batch:
            raise ValueError("contiguous cache batch dimension does not match q")
        return Shape(batch, n_heads, G, D, code, 0, int(k_cache.shape[1]), 0, 0)
    bs = int(k_cache.shape[1])
    if bs not in (16, 32):
        raise ValueError("paged pool must have 16- or 32-token blocks")
    if block_table.dim() != 2 or int(block_table.shape[0]) != batch:
        raise ValueError("block_table must be [batch, max_blocks_per_seq]")
    mbps = int(block_table.shape[1])
    return Shape(batch, n_heads, G, D, code, bs, mbps * bs, int(k_cache.shape[0]), mbps)


def rope_append_kv(q: Optional[torch.Tensor], k_new: torch.Tensor, v_new: torch.Tensor,
                   k_cache: torch.Tensor, v_cache: torch.Tensor, positions: torch.Tensor,
                   block_table: Optional[torch.Tensor] = None, base: float = 10000.0,
                   style: str = "interleaved",
                   q_rot: Optional[torch.Tensor] = None) -> Optional[torch.Tensor]:
    """RoPE on q and k_new at ``positions`` and the append of k_rot / v_new into
    the caches (in place).  Returns q_rot [B, H, D] float32 (None if q is None)."""
    lib = load_library()
    dev = k_cache.device
    B, G, D = int(k_new.shape[0]), int(k_new.shape[1]), int(k_new.shape[2])
    H = int(q.shape[1]) if q is not None else G
    shape = make_shape(B, H, k_cache, block_table)
    dt = k_cache.dtype
    if q is not None:
        _need(q, "q", dev, dt, (B, H, D))
    _need(k_new, "k_new", dev, dt, (B, G, D))
    _need(v_new, "v_new", dev, dt, (B, G, D))
    _need(k_cache, "k_cache", dev, dt)
    _need(v_cache, "v_cache", dev, dt, tuple(k_cache.shape))
    _need(positions, "positions", dev, torch.int32, (B,))
    if block_table is not None:
        _need(block_table, "block_table", dev, torch.int32)
    if style not in _STYLES:
        raise ValueError(f"style must be one of {sorted(_STYLES)}")
    if q is not None and q_rot is None:
        q_rot = torch.empty((B, H, D), dtype=torch.float32, device=dev)
    if q_rot is not None:
        _need(q_rot, "q_rot", dev, torch.float32, (B, H, D))
    _check(lib.rope_append_kv(ctypes.byref(shape), _ptr(q), _ptr(k_new), _ptr(v_new),
                              _ptr(q_rot) if q is not None else None, _ptr(k_cache),
                              _ptr(v_cache), _ptr(positions), _ptr(block_table),
                              float(base), _STYLES[style], _stream(dev)))
    return q_rot if q is not None else None


def _workspace(dev: torch.device, nbytes: int) -> Optional[torch.Tensor]:
    """A fresh workspace from torch's caching allocator, tied to the current
    stream (torch's allocator aligns blocks to at least 512 bytes)."""
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=dev)


def workspace_size(q_rot: torch.Tensor, k_cache: torch.Tensor,
                   block_table: Optional[torch.Tensor] = None,
                   max_seq_len: Optional[int] = None, n_query: int = 1,
                   options: Optional[Options] = None) -> int:
    """Workspace bytes of the decode call for q_rot [B, H, D] (n_query 1) or
    [B, T, H, D] (n_query T) with these options."""
    lib = load_library()
    B, H = int(q_rot.shape[0]), int(q_rot.shape[-2])
    shape = make_shape(B, H, k_cache, block_table)
    msl = shape.max_seq_len if max_seq_len is None else int(max_seq_len)
    return int(lib.gqa_decode_workspace_size_multi(ctypes.byref(shape), int(n_query), msl,
                                                   _options(options)))


def _scale_arg(scale: Optional[float]) -> float:
    """The scale passed to the library: 0 asks it for its default 1/sqrt(D)."""
    if scale is None:
        return 0.0
    if float(scale) == 0.0:
        raise ValueError("scale must be nonzero (None selects 1/sqrt(head_dim))")
    return float(scale)


def _outputs(lead, H, D, dev, out, lse, want_lse):
    if out is None:
        out = torch.empty((*lead, H, D), dtype=torch.float32, device=dev)
    _need(out, "out", dev, torch.float32, (*lead, H, D))
    if lse is None and want_lse:
        lse = torch.empty((*lead, H), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", dev, torch.float32, (*lead, H))
    return out, lse


def _attn_multi(shape, T, q_rot, k_cache, v_cache, k_scale, v_scale, seq_lens, block_table, msl,
                scale, out, lse, workspace, options, dev):
    """gqa_decode_attn_multi through the C ABI, with a per-call workspace
    unless the caller brings one."""
    lib = load_library()
    opts = _options(options)
    if workspace is None:
        nbytes = int(lib.gqa_decode_workspace_size_multi(ctypes.byref(shape), T, msl, opts))
        workspace = _workspace(dev, nbytes)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.gqa_decode_attn_multi(ctypes.byref(shape), T, _ptr(q_rot), _ptr(k_cache),
                                     _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _ptr(seq_lens),
                                     _ptr(block_table), msl, _scale_arg(scale), _ptr(out),
                                     _ptr(lse), _ptr(workspace), wbytes, opts, _stream(dev)))



def gqa_decode_attn(q_rot: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                    seq_lens: torch.Tensor, block_table: Optional[torch.Tensor] = None,
                    scale: Optional[float] = None, max_seq_len: Optional[int] = None,
                    out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None, want_lse: bool = True,
                    options: Optional[Options] = None
                    ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """softmax(q K^T * scale) V per (b, h) over the first seq_lens[b] cached
    tokens (fp32 or bf16 cache).  Returns (out [B, H, D] float32, lse [B, H]
    float32 natural log).

    ``max_seq_len`` is the host-side bound on seq_lens used to plan the grid
    (default: the cache capacity); ``scale`` None lets the library use
    1/sqrt(D).  With ``options`` the call goes through gqa_decode_attn_multi
    (one new token), which takes them."""
    lib = load_library()
    dev = k_cache.device
    B, H, D = (int(x) for x in q_rot.shape)
    shape = make_shape(B, H, k_cache, block_table)
    _need(q_rot, "q_rot", dev, torch.float32, (B, H, D))
    _need(k_cache, "k_cache", dev)
    _need(v_cache, "v_cache", dev, k_cache.dtype, tuple(k_cache.shape))
    _need(seq_lens, "seq_lens", dev, torch.int32, (B,))
    if block_table is not None:
        _need(block_table, "block_table", dev, torch.int32)
    if int(k_cache.shape[3]) != D:
        raise ValueError("head_dim of q_rot and cache differ")
    msl = shape.max_seq_len if max_seq_len is None else int(max_seq_len)
    out, lse = _outputs((B,), H, D, dev, out, lse, want_lse)
    if options is not None:
        _attn_multi(shape, 1, q_rot, k_cache, v_cache, None, None, seq_lens, block_table, msl,
                    scale, out, lse, workspace, options, dev)
        return out, lse
    if workspace is None:
        workspace = _workspace(dev, int(lib.gqa_decode_workspace_size(ctypes.byref(shape), msl)))
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.gqa_decode_attn(ctypes.byref(shape), _ptr(q_rot), _ptr(k_cache), _ptr(v_cache),
                               _ptr(seq_lens), _ptr(block_table), msl, _scale_arg(scale),
                               _ptr(out), _ptr(lse), _ptr(workspace), wbytes, _stream(dev)))
    return out, lse



def v_cache_shape_int8(k_cache: torch.Tensor, paged: bool) -> Tuple[int, ...]:
    """Shape of the INT8 V cache that goes with an int8 K cache: per 16-token
    group and head, V transposed ([.., G, D, 16] against K's [.., G, 16, D])."""
    if paged and k_cache.dim() == 4:
        nb, G, _, D = (int(x) for x in k_cache.shape)
        return (nb, G, D, 16)
    a, n, G, _, D = (int(x) for x in k_cache.shape)
    return (a, n, G, D, 16)


def _check_scales(k_scale, v_scale, G, dev):
    _need(k_scale, "k_scale", dev, torch.float32, (G,))
    _need(v_scale, "v_scale", dev, torch.float32, (G,))


def rope_append_kv_int8(q: Optional[torch.Tensor], k_new: torch.Tensor, v_new: torch.Tensor,
                        k_cache: torch.Tensor, v_cache: torch.Tensor, k_scale: torch.Tensor,
                        v_scale: torch.Tensor, positions: torch.Tensor,
                        block_table: Optional[torch.Tensor] = None, base: float = 10000.0,
                        style: str = "interleaved",
                        q_rot: Optional[torch.Tensor] = None) -> Optional[torch.Tensor]:
    """rope_append_kv into an INT8 cache: bf16 q / k_new / v_new, int8 K cache
    [B, S_max/16, G, 16, D] (or pool [NB, G, 16, D]) and V cache
    [B, S_max/16, G, D, 16] (or [NB, G, D, 16]), per-KV-head fp32 scales."""
    lib = load_library()
    dev = k_cache.device
    B, G, D = int(k_new.shape[0]), int(k_new.shape[1]), int(k_new.shape[2])
    H = int(q.shape[1]) if q is not None else G
    shape = make_shape(B, H, k_cache, block_table)
    if q is not None:
        _need(q, "q", dev, torch.bfloat16, (B, H, D))
    _need(k_new, "k_new", dev, torch.bfloat16, (B, G, D))
    _need(v_new, "v_new", dev, torch.bfloat16, (B, G, D))
    _need(k_cache, "k_cache", dev, torch.int8)
    _need(v_cache, "v_cache", dev, torch.int8, v_cache_shape_int8(k_cache, block_table is not None))
    _check_scales(k_scale, v_scale, G, dev)
    _need(positions, "positions", dev, torch.int32, (B,))
    if block_table is not None:
        _need(block_table, "block_table", dev, torch.int32)
    if style not in _STYLES:
        raise ValueError(f"style must be one of {sorted(_STYLES)}")
    if q is not None and q_rot is None:
        q_rot = torch.empty((B, H, D), dtype=torch.float32, device=dev)
    if q_rot is not None:
        _need(q_rot, "q_rot", dev, torch.float32, (B, H, D))
    _check(lib.rope_append_kv_int8(ctypes.byref(shape), _ptr(q), _ptr(k_new), _ptr(v_new),
                                   _ptr(q_rot) if q is not None else None, _ptr(k_cache),
                                   _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _ptr(positions),
                                   _ptr(block_table), float(base), _STYLES[style], _stream(dev)))
    return q_rot if q is not None else None


def gqa_decode_attn_int8(q_rot: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                         k_scale: torch.Tensor, v_scale: torch.Tensor, seq_lens: torch.Tensor,
                         block_table: Optional[torch.Tensor] = None,
                         scale: Optional[float] = None, max_seq_len: Optional[int] = None,
                         out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None, want_lse: bool = True,
                         options: Optional[Options] = None
                         ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """gqa_decode_attn over an INT8 cache (layouts as rope_append_kv_int8)."""
    lib = load_library()
    dev = k_cache.device
    B, H, D = (int(x) for x in q_rot.shape)
    shape = make_shape(B, H, k_cache, block_table)
    _need(q_rot, "q_rot", dev, torch.float32, (B, H, D))
    _need(k_cache, "k_cache", dev, torch.int8)
    _need(v_cache, "v_cache", dev, torch.int8, v_cache_shape_int8(k_cache, block_table is not None))
    _check_scales(k_scale, v_scale, shape.n_kv_heads, dev)
    _need(seq_lens, "seq_lens", dev, torch.int32, (B,))
    if block_table is not None:
        _need(block_table, "block_table", dev, torch.int32)
    if shape.head_dim != D:
        raise ValueError("head_dim of q_rot and cache differ")
    msl = shape.max_seq_len if max_seq_len is None else int(max_seq_len)
    out, lse = _outputs((B,), H, D, dev, out, lse, want_lse)
    if options is not None:
        _attn_multi(shape, 1, q_rot, k_cache, v_cache, k_scale, v_scale, seq_lens, block_table,
                    msl, scale, out, lse, workspace, options, dev)
        return out, lse
    if workspace is None:
        workspace = _workspace(dev, int(lib.gqa_decode_workspace_size(ctypes.byref(shape), msl)))
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.gqa_decode_attn_int8(ctypes.byref(shape), _ptr(q_rot), _ptr(k_cache),
                                    _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _ptr(seq_lens),
                                    _ptr(block_table), msl, _scale_arg(scale), _ptr(out),
                                    _ptr(lse), _ptr(workspace), wbytes, _stream(dev)))
    return out, lse



def _check_rings(k_recent, v_recent, B, G, D, dev):
    """The bf16 rings [B, W, G, D] of a mixed-precision cache; returns W."""
    _need(k_recent, "k_recent", dev, torch.bfloat16)
    if k_recent.dim() != 4 or tuple(k_recent.shape[::2]) != (B, G) or int(k_recent.shape[3]) != D:
        raise ValueError(f"k_recent: expected [B={B}, W, G={G}, D={D}], got {tuple(k_recent.shape)}")
    _need(v_recent, "v_recent", dev, torch.bfloat16, tuple(k_recent.shape))
    return int(k_recent.shape[1])


def rope_append_kv_mixed(q: Optional[torch.Tensor], k_new: torch.Tensor, v_new: torch.Tensor,
                         k_cache: torch.Tensor, v_cache: torch.Tensor, k_scale: torch.Tensor,
                         v_scale: torch.Tensor, k_recent: torch.Tensor, v_recent: torch.Tensor,
                         positions: torch.Tensor, block_table: Optional[torch.Tensor] = None,
                         base: float = 10000.0, style: str = "interleaved",
                         q_rot: Optional[torch.Tensor] = None) -> Optional[torch.Tensor]:
    """rope_append_kv into a mixed-precision cache: the W newest tokens in the
    bf16 rings k_recent / v_recent [B, W, G, D] (token p in row p mod W), the
    older ones in the INT8 cache (layouts and scales as rope_append_kv_int8).
    The token that leaves the ring is quantised into the INT8 cache."""
    lib = load_library()
    dev = k_cache.device
    B, G, D = int(k_new.shape[0]), int(k_new.shape[1]), int(k_new.shape[2])
    H = int(q.shape[1]) if q is not None else G
    shape = make_shape(B, H, k_cache, block_table)
    if q is not None:
        _need(q, "q", dev, torch.bfloat16, (B, H, D))
    _need(k_new, "k_new", dev, torch.bfloat16, (B, G, D))
    _need(v_new, "v_new", dev, torch.bfloat16, (B, G, D))
    _need(k_cache, "k_cache", dev, torch.int8)
    _need(v_cache, "v_cache", dev, torch.int8, v_cache_shape_int8(k_cache, block_table is not None))
    _check_scales(k_scale, v_scale, G, dev)
    window = _check_rings(k_recent, v_recent, B, G, D, dev)
    _need(positions, "positions", dev, torch.int32, (B,))
    if block_table is not None:
        _need(block_table, "block_table", dev, torch.int32)
    if style not in _STYLES:
        raise ValueError(f"style must be one of {sorted(_STYLES)}")
    if q is not None and q_rot is None:
        q_rot = torch.empty((B, H, D), dtype=torch.float32, device=dev)
    if q_rot is not None:
        _need(q_rot, "q_rot", dev, torch.float32, (B, H, D))
    _check(lib.rope_append_kv_mixed(ctypes.byref(shape), window, _ptr(q), _ptr(k_new),
                                    _ptr(v_new), _ptr(q_rot) if q is not None else None,
                                    _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
                                    _ptr(k_recent), _ptr(v_recent), _ptr(positions),
                                    _ptr(block_table), float(base), _STYLES[style], _stream(dev)))
    return q_rot if q is not None else None


def gqa_decode_attn_mixed(q_rot: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                          k_scale: torch.Tensor, v_scale: torch.Tensor, k_recent: torch.Tensor,
                          v_recent: torch.Tensor, seq_lens: torch.Tensor,
                          block_table: Optional[torch.Tensor] = None,
                          scale: Optional[float] = None, max_seq_len: Optional[int] = None,
                          out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None, want_lse: bool = True,
                          options: Optional[Options] = None
                          ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """gqa_decode_attn over a mixed-precision cache (rope_append_kv_mixed):
    the last W of each sequence's tokens from the bf16 rings, the rest from
    the INT8 cache."""
    lib = load_library()
    dev = k_cache.device
    B, H, D = (int(x) for x in q_rot.shape)
    shape = make_shape(B, H, k_cache, block_table)
    _need(q_rot, "q_rot", dev, torch.float32, (B, H, D))
    _need(k_cache, "k_cache", dev, torch.int8)
    _need(v_cache, "v_cache", dev, torch.int8, v_cache_shape_int8(k_cache, block_table is not None))
    _check_scales(k_scale, v_scale, shape.n_kv_heads, dev)
    window = _check_rings(k_recent, v_recent, B, shape.n_kv_heads, D, dev)
    _need(seq_lens, "seq_lens", dev, torch.int32, (B,))
    if block_table is not None:
        _need(block_table, "block_table", dev, torch.int32)
    if shape.head_dim != D:
        raise ValueError("head_dim of q_rot and cache differ")
    msl = shape.max_seq_len if max_seq_len is None else int(max_seq_len)
    out, lse = _outputs((B,), H, D, dev, out, lse, want_lse)
    opts = _options(options)
    if workspace is None:
        workspace = _workspace(dev, int(lib.gqa_decode_workspace_size_mixed(
            ctypes.byref(shape), window, msl, opts)))
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.gqa_decode_attn_mixed(ctypes.byref(shape), window, _ptr(q_rot), _ptr(k_cache),
                                     _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
                                     _ptr(k_recent), _ptr(v_recent), _ptr(seq_lens),
                                     _ptr(block_table), msl, _scale_arg(scale), _ptr(out),
                                     _ptr(lse), _ptr(workspace), wbytes, opts, _stream(dev)))
    return out, lse


def workspace_size_mixed(batch: int, n_heads: int, k_cache: torch.Tensor, window: int,
                         block_table: Optional[torch.Tensor] = None,
                         max_seq_len: Optional[int] = None,
                         options: Optional[Options] = None) -> int:
    """Workspace bytes gqa_decode_attn_mixed takes."""
    shape = make_shape(batch, n_heads, k_cache, block_table)
    msl = shape.max_seq_len if max_seq_len is None else int(max_seq_len)
    return int(load_library().gqa_decode_workspace_size_mixed(ctypes.byref(shape), int(window),
                                                              msl, _options(options)))


def _multi_cache_checks(k_cache, v_cache, k_scale, v_scale, G, dev, paged):
    """Input dtype of the multi-token calls; checks the caches and scales."""
    if k_cache.dtype == torch.int8:
        _need(k_cache, "k_cache", dev, torch.int8)
        _need(v_cache, "v_cache", dev, torch.int8, v_cache_shape_int8(k_cache, paged))
        if k_scale is None or v_scale is None:
            raise ValueError("an int8 cache needs k_scale and v_scale")
        _check_scales(k_scale, v_scale, G, dev)
        return torch.bfloat16
    if k_scale is not None or v_scale is not None:
        raise ValueError("k_scale / v_scale belong to int8 caches only")
    _need(k_cache, "k_cache", dev)
    _need(v_cache, "v_cache", dev, k_cache.dtype, tuple(k_cache.shape))
    return k_cache.dtype


def rope_append_kv_multi(q: Optional[torch.Tensor], k_new: torch.Tensor, v_new: torch.Tensor,
                         k_cache: torch.Tensor, v_cache: torch.Tensor, positions: torch.Tensor,
                         block_table: Optional[torch.Tensor] = None,
                         k_scale: Optional[torch.Tensor] = None,
                         v_scale: Optional[torch.Tensor] = None, base: float = 10000.0,
                         style: str = "interleaved",
                         q_rot: Optional[torch.Tensor] = None) -> Optional[torch.Tensor]:
    """T new tokens per sequence: q [B, T, H, D], k_new / v_new [B, T, G, D];
    token t of sequence b is rotated at positions[b] + t and appended there.
    Returns q_rot [B, T, H, D] float32 (None if q is None).  int8 caches take
    bf16 inputs and their per-head scales, other caches inputs of their dtype."""
    lib = load_library()
    dev = k_cache.device
    B, T, G, D = (int(x) for x in k_new.shape)
    H = int(q.shape[2]) if q is not None else G
    shape = make_shape(B, H, k_cache, block_table)
    dt = _multi_cache_checks(k_cache, v_cache, k_scale, v_scale, G, dev, block_table is not None)
    if q is not None:
        _need(q, "q", dev, dt, (B, T, H, D))
    _need(k_new, "k_new", dev, dt, (B, T, G, D))
    _need(v_new, "v_new", dev, dt, (B, T, G, D))
    _need(positions, "positions", dev, torch.int32, (B,))
    if block_table is not None:
        _need(block_table, "block_table", dev, torch.int32)
    if style not in _STYLES:
        raise ValueError(f"style must be one of {sorted(_STYLES)}")
    if q is not None and q_rot is None:
        q_rot = torch.empty((B, T, H, D), dtype=torch.float32, device=dev)
    if q_rot is not None:
        _need(q_rot, "q_rot", dev, torch.float32, (B, T, H, D))
    _check(lib.rope_append_kv_multi(ctypes.byref(shape), T, _ptr(q), _ptr(k_new), _ptr(v_new),
                                    _ptr(q_rot) if q is not None else None, _ptr(k_cache),
                                    _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _ptr(positions),
                                    _ptr(block_table), float(base), _STYLES[style], _stream(dev)))
    return q_rot if q is not None else None


def gqa_decode_attn_multi(q_rot: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                          seq_lens: torch.Tensor, block_table: Optional[torch.Tensor] = None,
                          k_scale: Optional[torch.Tensor] = None,
                          v_scale: Optional[torch.Tensor] = None,
                          scale: Optional[float] = None, max_seq_len: Optional[int] = None,
                          out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None, want_lse: bool = True,
                          options: Optional[Options] = None
                          ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Attention of T new tokens per sequence, q_rot [B, T, H, D]: with
    L = seq_lens[b] (the new tokens included), query t attends the tokens
    j < L - T + 1 + t.  Returns (out [B, T, H, D], lse [B, T, H])."""
    dev = k_cache.device
    B, T, H, D = (int(x) for x in q_rot.shape)
    shape = make_shape(B, H, k_cache, block_table)
    _need(q_rot, "q_rot", dev, torch.float32, (B, T, H, D))
    _multi_cache_checks(k_cache, v_cache, k_scale, v_scale, shape.n_kv_heads, dev,
                        block_table is not None)
    _need(seq_lens, "seq_lens", dev, torch.int32, (B,))
    if block_table is not None:
        _need(block_table, "block_table", dev, torch.int32)
    if shape.head_dim != D:
        raise ValueError("head_dim of q_rot and cache differ")
    msl = shape.max_seq_len if max_seq_len is None else int(max_seq_len)
    out, lse = _outputs((B, T), H, D, dev, out, lse, want_lse)
    _attn_multi(shape, T, q_rot, k_cache, v_cache, k_scale, v_scale, seq_lens, block_table, msl,
                scale, out, lse, workspace, options, dev)
    return out, lse



def gqa_decode_step(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                    k_cache: torch.Tensor, v_cache: torch.Tensor, positions: torch.Tensor,
                    block_table: Optional[torch.Tensor] = None, base: float = 10000.0,
                    style: str = "interleaved", scale: Optional[float] = None,
                    max_seq_len: Optional[int] = None, q_rot: Optional[torch.Tensor] = None,
                    out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None, want_lse: bool = True,
                    options: Optional[Options] = None, k_scale: Optional[torch.Tensor] = None,
                    v_scale: Optional[torch.Tensor] = None
                    ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """The decode step in one call (gqa_decode_step): rope_append_kv, then
    attention over positions[b] + 1 tokens, for a bf16 cache (or an INT8
    cache with ``k_scale`` / ``v_scale``: gqa_decode_step_int8) with up to 32
    (INT8: 16) query heads per KV head.  q [B, H, D], k_new / v_new [B, G, D] bf16;
    ``q_rot`` (optional, [B, H, D] float32) receives the rotated q.
    Returns (out [B, H, D], lse [B, H]).

    With q [B, T, H, D] and k_new / v_new [B, T, G, D] (bf16 cache, T <= 16
    new tokens, T x query heads per KV head <= 32): gqa_decode_step_multi,
    rope_append_kv_multi then attention over positions[b] + T tokens;
    q_rot, out [B, T, H, D], lse [B, T, H]."""
    lib = load_library()
    dev = k_cache.device
    multi = q.dim() == 4
    if multi:
        B, T, H, D = (int(x) for x in q.shape)
        G = int(k_new.shape[2])
    else:
        B, H, D = (int(x) for x in q.shape)
        T, G = 1, int(k_new.shape[1])
    lead = (B, T) if multi else (B,)
    shape = make_shape(B, H, k_cache, block_table)
    int8 = k_cache.dtype == torch.int8
    if multi and int8:
        raise ValueError("several new tokens per sequence need a bf16 cache")
    dt = _multi_cache_checks(k_cache, v_cache, k_scale, v_scale, G, dev, block_table is not None)
    _need(q, "q", dev, dt, lead + (H, D))
    _need(k_new, "k_new", dev, dt, lead + (G, D))
    _need(v_new, "v_new", dev, dt, lead + (G, D))
    _need(positions, "positions", dev, torch.int32, (B,))
    if block_table is not None:
        _need(block_table, "block_table", dev, torch.int32)
    if q_rot is not None:
        _need(q_rot, "q_rot", dev, torch.float32, lead + (H, D))
    if style not in _STYLES:
        raise ValueError(f"style must be one of {sorted(_STYLES)}")
    msl = shape.max_seq_len if max_seq_len is None else int(max_seq_len)
    out, lse = _outputs(lead, H, D, dev, out, lse, want_lse)
    opts = _options(options)
    if workspace is None:
        nbytes = int(lib.gqa_decode_workspace_size_multi(ctypes.byref(shape), T, msl, opts))
        workspace = _workspace(dev, nbytes)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if multi:
        _check(lib.gqa_decode_step_multi(
            ctypes.byref(shape), T, _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
            _ptr(v_cache), _ptr(positions), _ptr(block_table), msl, float(base), _STYLES[style],
            _scale_arg(scale), _ptr(q_rot), _ptr(out), _ptr(lse), _ptr(workspace), wbytes, opts,
            _stream(dev)))
    elif int8:
        _check(lib.gqa_decode_step_int8(
            ctypes.byref(shape), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
            _ptr(k_scale), _ptr(v_scale), _ptr(positions), _ptr(block_table), msl, float(base),
            _STYLES[style], _scale_arg(scale), _ptr(q_rot), _ptr(out), _ptr(lse),
            _ptr(workspace), wbytes, opts, _stream(dev)))
    else:
        _check(lib.gqa_decode_step(ctypes.byref(shape), _ptr(q), _ptr(k_new), _ptr(v_new),
                                   _ptr(k_cache), _ptr(v_cache), _ptr(positions),
                                   _ptr(block_table), msl, float(base), _STYLES[style],
                                   _scale_arg(scale), _ptr(q_rot), _ptr(out), _ptr(lse),
                                   _ptr(workspace), wbytes, opts, _stream(dev)))
    return out, lse


def gqa_decode_attn_noalloc(q_rot: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                            seq_lens: torch.Tensor, block_table: Optional[torch.Tensor] = None,
                            k_scale: Optional[torch.Tensor] = None,
                            v_scale: Optional[torch.Tensor] = None,
                            scale: Optional[float] = None, max_seq_len: Optional[int] = None,
                            out: Optional[torch.Tensor] = None,
                            lse: Optional[torch.Tensor] = None, want_lse: bool = True,
                            options: Optional[Options] = None
                            ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """gqa_decode_attn_multi through gqa_decode_attn_multi_noalloc: the split
    partials live in the library's own device array (at most
    NOALLOC_SCRATCH_BYTES), so with ``out`` (and ``lse``) given nothing is
    allocated.  q_rot [B, T, H, D]; calls overlapping on one device race."""
    lib = load_library()
    dev = k_cache.device
    B, T, H, D = (int(x) for x in q_rot.shape)
    shape = make_shape(B, H, k_cache, block_table)
    _need(q_rot, "q_rot", dev, torch.float32, (B, T, H, D))
    _multi_cache_checks(k_cache, v_cache, k_scale, v_scale, shape.n_kv_heads, dev,
                        block_table is not None)
    _need(seq_lens, "seq_lens", dev, torch.int32, (B,))
    if block_table is not None:
        _need(block_table, "block_table", dev, torch.int32)
    if shape.head_dim != D:
        raise ValueError("head_dim of q_rot and cache differ")
    msl = shape.max_seq_len if max_seq_len is None else int(max_seq_len)
    out, lse = _outputs((B, T), H, D, dev, out, lse, want_lse)
    _check(lib.gqa_decode_attn_multi_noalloc(
        ctypes.byref(shape), T, _ptr(q_rot), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
        _ptr(v_scale), _ptr(seq_lens), _ptr(block_table), msl, _scale_arg(scale), _ptr(out),
        _ptr(lse), _options(options), _stream(dev)))
    return out, lse


def gqa_prefill_attn(q_rot: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                     seq_lens: torch.Tensor, block_table: Optional[torch.Tensor] = None,
                     scale: Optional[float] = None, max_seq_len: Optional[int] = None,
                     out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                     want_lse: bool = True, options: Optional[Options] = None,
                     workspace: Optional[torch.Tensor] = None,
                     k_scale: Optional[torch.Tensor] = None,
                     v_scale: Optional[torch.Tensor] = None
                     ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Causal attention of T new tokens per sequence (a prompt or a chunk of
    one, already appended), q_rot [B, T, H, D], over a bf16 cache, or an
    INT8 cache with its per-head ``k_scale`` / ``v_scale``; query t attends
    the tokens j < seq_lens[b] - T + 1 + t.  q and P enter the matrix cores
    as bf16 (fp16 on an INT8 cache).  ``options`` may carry split_tokens (a
    multiple of 32), a prefill dispatch order and timing events.  The
    key-split partials go to ``workspace`` or to a per-call allocation of the
    size the library asks for.  Returns (out [B, T, H, D], lse [B, T, H])."""
    lib = load_library()
    dev = k_cache.device
    B, T, H, D = (int(x) for x in q_rot.shape)
    shape = make_shape(B, H, k_cache, block_table)
    _need(q_rot, "q_rot", dev, torch.float32, (B, T, H, D))
    i8 = k_cache.dtype == torch.int8
    if i8:
        _need(v_cache, "v_cache", dev, torch.int8,
              v_cache_shape_int8(k_cache, block_table is not None))
        _check_scales(k_scale, v_scale, shape.n_kv_heads, dev)
    else:
        if k_scale is not None or v_scale is not None:
            raise ValueError("scales are only for INT8 caches")
        _need(k_cache, "k_cache", dev, torch.bfloat16)
        _need(v_cache, "v_cache", dev, torch.bfloat16, tuple(k_cache.shape))
    _need(seq_lens, "seq_lens", dev, torch.int32, (B,))
    if block_table is not None:
        _need(block_table, "block_table", dev, torch.int32)
    if shape.head_dim != D:
        raise ValueError("head_dim of q_rot and cache differ")
    msl = shape.max_seq_len if max_seq_len is None else int(max_seq_len)
    out, lse = _outputs((B, T), H, D, dev, out, lse, want_lse)
    opts = _options(options)
    if workspace is None:
        nbytes = int(lib.gqa_prefill_workspace_size(ctypes.byref(shape), T, msl, opts))
        workspace = _workspace(dev, nbytes)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if i8:
        _check(lib.gqa_prefill_attn_int8(ctypes.byref(shape), T, _ptr(q_rot), _ptr(k_cache),
                                         _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
                                         _ptr(seq_lens), _ptr(block_table), msl,
                                         _scale_arg(scale), _ptr(out), _ptr(lse),
                                         _ptr(workspace), wbytes, opts, _stream(dev)))
        return out, lse
    _check(lib.gqa_prefill_attn(ctypes.byref(shape), T, _ptr(q_rot), _ptr(k_cache), _ptr(v_cache),
                                _ptr(seq_lens), _ptr(block_table), msl, _scale_arg(scale),
                                _ptr(out), _ptr(lse), _ptr(workspace), wbytes, opts,
                                _stream(dev)))
    return out, lse


def prefill_workspace_size(batch: int, n_heads: int, n_query: int, k_cache: torch.Tensor,
                           block_table: Optional[torch.Tensor] = None,
                           max_seq_len: Optional[int] = None,
                           options: Optional[Options] = None) -> int:
    """Bytes of key-split workspace gqa_prefill_attn would take (0: no split)."""
    shape = make_shape(batch, n_heads, k_cache, block_table)
    msl = shape.max_seq_len if max_seq_len is None else int(max_seq_len)
    return int(load_library().gqa_prefill_workspace_size(ctypes.byref(shape), int(n_query), msl,
                                                         _options(options)))


def get_plan(batch: int, n_heads: int, k_cache: torch.Tensor,
             block_table: Optional[torch.Tensor] = None, max_seq_len: Optional[int] = None,
             n_query: int = 1, options: Optional[Options] = None):
    """{'split_tokens', 'n_splits', 'kernel', 'workgroups'} the library would use."""
    shape = make_shape(batch, n_heads, k_cache, block_table)
    msl = shape.max_seq_len if max_seq_len is None else int(max_seq_len)
    arr = (ctypes.c_int32 * 4)()
    _check(load_library().kvd_get_plan_multi(ctypes.byref(shape), int(n_query), msl,
                                             _options(options), arr))
    return {"split_tokens": arr[0], "n_splits": arr[1],
            "kernel": _KERNEL_NAMES[arr[2]], "workgroups": arr[3]}



PROBE_CHUNKED, PROBE_NONTEMPORAL, PROBE_LDS = 1, 2, 4


def read_probe(buf: torch.Tensor, n_workgroups: int, unroll: int = 8, mode: int = 0,
               sink: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Launch the streaming-read probe over all bytes of ``buf`` (measurement
    only); ``mode`` ORs PROBE_CHUNKED, PROBE_NONTEMPORAL and PROBE_LDS.
    Returns the sink tensor."""
    if sink is None or sink.numel() < n_workgroups:
        sink = torch.empty(n_workgroups, dtype=torch.int32, device=buf.device)
    nbytes = buf.numel() * buf.element_size()
    _check(load_library().kvd_read_probe(_ptr(buf), nbytes, _ptr(sink), int(n_workgroups),
                                         int(unroll), int(mode), _stream(buf.device)))
    return sink
