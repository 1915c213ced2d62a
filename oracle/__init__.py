"""fp64 CPU oracle for the GQA decode step (RoPE, KV-cache append, attention).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  It never
imports the GPU package and the GPU package never imports it; the two share
no code.  Inputs reach both sides from the seeded workload generators, which
hold no arithmetic of the method.

Contents
--------
* ``liboracle.so`` (from ``kvoracle.c``): the decode step in plain C loops,
  fp64 throughout -- RoPE rotation, append at the slot given by the position,
  textbook two-pass softmax attention with the GQA head mapping g = h / n_rep.
* ``full_causal``: an independently written NumPy recompute of causal
  attention from scratch (RoPE through complex multiplication), used to pin
  the decode loop.
* ``merge``: the log-sum-exp merge of attention over disjoint token sets.

INT8 caches ([KVGR] §4.3: K and V stored as 8-bit integers with
quantisation parameters calibrated per attention head): dtype ``"i8"``.  q,
k_new and v_new are then bf16; the caches hold codes in [-127, 127] with one
fp32 scale per KV head for K (``k_scale``) and one for V (``v_scale``).  A
new element x is stored as the code nearest to x / scale (ties to even,
saturating); attention reads scale * code.  Tokens are grouped by 16 and
each group holds, per KV head, the 16 K rows and the V block transposed
(``Geometry.cache_shape`` / ``Geometry.v_cache_shape``).

Mixed precision ([KVGR] §4.3 names caches that keep the most recent tokens at
high precision and quantise the older history): the W newest tokens of each
sequence sit in bf16 rings ``k_recent`` / ``v_recent`` [B, W, G, D] (token p
in row p mod W), every older token in an INT8 cache as above.  The append of
the token at position P first moves token P - W (when P >= W) from its ring
row into the INT8 cache as codes of its bf16 values, then writes the new
token into that row (``rope_append_mixed``); attention reads the last W of
the L attended tokens from the rings (``decode_attn_mixed``).

Arrays: bf16 data are passed as ``uint16`` bit patterns; fp32 as ``float32``;
fp64 as ``float64``.  Pages cited by title:
  [KVGR] "Transformer推理核心：KV Cache、GQA与RoPE原理与工程实践"
  [SA4]  "4. 自注意力机制推理：单步计算、KV Cache的引入与原理"
  [OPT]  "Transformer架构优化实战2026：注意力机制、KV Cache与推理加速完整指南"
"""
import ctypes
import os

import numpy as np

from .build import LIB, build

F64, F32, BF16, I8 = 0, 1, 2, 3
INTERLEAVED, HALF = 0, 1

_DTYPE_CODE = {"f64": F64, "f32": F32, "bf16": BF16, "i8": I8}
_NP_STORAGE = {F64: np.float64, F32: np.float32, BF16: np.uint16, I8: np.int8}
_NP_INPUT = {F64: np.float64, F32: np.float32, BF16: np.uint16, I8: np.uint16}
_STYLE_CODE = {"interleaved": INTERLEAVED, "half": HALF}


class _Shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "n_heads", "n_kv_heads", "head_dim", "dtype", "block_size",
        "max_seq_len", "num_blocks", "max_blocks_per_seq")]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        lib = ctypes.CDLL(LIB)
        P = ctypes.c_void_p
        lib.kvo_round_to_bf16.restype = ctypes.c_double
        lib.kvo_round_to_bf16.argtypes = [ctypes.c_double]
        lib.kvo_bf16_bits.restype = ctypes.c_uint16
        lib.kvo_bf16_bits.argtypes = [ctypes.c_double]
        lib.kvo_quantize_i8.restype = ctypes.c_int
        lib.kvo_quantize_i8.argtypes = [ctypes.c_double, ctypes.c_double]
        lib.kvo_theta.restype = ctypes.c_double
        lib.kvo_theta.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_double]
        lib.kvo_rope_rotate.restype = None
        lib.kvo_rope_rotate.argtypes = [P, P, ctypes.c_int, ctypes.c_double,
                                        ctypes.c_double, ctypes.c_int]
        lib.kvo_rope_append.restype = ctypes.c_int
        lib.kvo_rope_append.argtypes = [ctypes.POINTER(_Shape), P, P, P, P, P, P,
                                        P, P, ctypes.c_double, ctypes.c_int]
        lib.kvo_rope_append_i8.restype = ctypes.c_int
        lib.kvo_rope_append_i8.argtypes = [ctypes.POINTER(_Shape), P, P, P, P, P, P, P, P,
                                           P, P, ctypes.c_double, ctypes.c_int]
        lib.kvo_decode_attn_i8.restype = ctypes.c_int
        lib.kvo_decode_attn_i8.argtypes = [ctypes.POINTER(_Shape), P, P, P, P, P, P, P,
                                           ctypes.c_double, P, P, P, ctypes.c_int]
        lib.kvo_decode_attn_units_i8.restype = ctypes.c_int
        lib.kvo_decode_attn_units_i8.argtypes = [ctypes.POINTER(_Shape), P, P, P, P, P, P,
                                                 P, ctypes.c_double, P, P, ctypes.c_int64,
                                                 P, P, ctypes.c_int]
        lib.kvo_rope_append_mq.restype = ctypes.c_int
        lib.kvo_rope_append_mq.argtypes = [ctypes.POINTER(_Shape), ctypes.c_int, P, P, P, P, P,
                                           P, P, P, P, P, ctypes.c_double, ctypes.c_int]
        lib.kvo_decode_attn_mq.restype = ctypes.c_int
        lib.kvo_decode_attn_mq.argtypes = [ctypes.POINTER(_Shape), ctypes.c_int, P, P, P, P, P,
                                           P, P, ctypes.c_double, P, P, P, ctypes.c_int]
        lib.kvo_decode_attn_units_mq.restype = ctypes.c_int
        lib.kvo_decode_attn_units_mq.argtypes = [ctypes.POINTER(_Shape), ctypes.c_int, P, P, P,
                                                 P, P, P, P, ctypes.c_double, P, P,
                                                 ctypes.c_int64, P, P, ctypes.c_int]
        lib.kvo_rope_append_mixed.restype = ctypes.c_int
        lib.kvo_rope_append_mixed.argtypes = [ctypes.POINTER(_Shape), ctypes.c_int, P, P, P, P,
                                              P, P, P, P, P, P, P, P, ctypes.c_double,
                                              ctypes.c_int]
        lib.kvo_decode_attn_mixed.restype = ctypes.c_int
        lib.kvo_decode_attn_mixed.argtypes = [ctypes.POINTER(_Shape), ctypes.c_int, P, P, P, P,
                                              P, P, P, P, P, ctypes.c_double, P, P,
                                              ctypes.c_int64, P, P, ctypes.c_int]
        lib.kvo_decode_attn.restype = ctypes.c_int
        lib.kvo_decode_attn.argtypes = [ctypes.POINTER(_Shape), P, P, P, P, P,
                                        ctypes.c_double, P, P, P, ctypes.c_int]
        lib.kvo_decode_attn_units.restype = ctypes.c_int
        lib.kvo_decode_attn_units.argtypes = [ctypes.POINTER(_Shape), P, P, P, P,
                                              P, ctypes.c_double, P, P,
                                              ctypes.c_int64, P, P, ctypes.c_int]
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _need(a, dtype, name, shape=None):
    if not isinstance(a, np.ndarray) or a.dtype != dtype or not a.flags.c_contiguous:
        raise TypeError(f"{name}: expected a C-contiguous {np.dtype(dtype).name} array")
    if shape is not None and tuple(a.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {a.shape} != {shape}")
    return a


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


class Geometry:
    """Shape of one decode problem, as the oracle sees it.

    Contiguous caches are ``[B, S_max, G, D]``; paged pools are
    ``[num_blocks, block_size, G, D]`` with an int32 table
    ``[B, max_blocks_per_seq]`` ([OPT] §四 PagedKVCache; [KVGR] §4.1).
    INT8 caches are grouped by 16 tokens, per head: K ``[B, S_max/16, G, 16, D]``
    or ``[num_blocks, G, 16, D]``, V ``[B, S_max/16, G, D, 16]`` or
    ``[num_blocks, G, D, 16]``; 32-token blocks hold two groups
    (``[num_blocks, 2, G, 16, D]``, ``[num_blocks, 2, G, D, 16]``).
    """

    def __init__(self, batch, n_heads, n_kv_heads, head_dim, dtype="bf16",
                 max_seq_len=None, block_size=0, num_blocks=0, max_blocks_per_seq=0):
        if n_heads % n_kv_heads:
            raise ValueError("n_heads must be a multiple of n_kv_heads")  # [OPT] §六 assert
        self.batch, self.n_heads, self.n_kv_heads, self.head_dim = batch, n_heads, n_kv_heads, head_dim
        self.dtype = dtype
        self.block_size, self.num_blocks = block_size, num_blocks
        self.max_blocks_per_seq = max_blocks_per_seq
        if block_size:
            max_seq_len = max_blocks_per_seq * block_size
        self.max_seq_len = max_seq_len
        if dtype == "i8" and (max_seq_len % 16 or block_size % 16):
            raise ValueError("INT8 caches group tokens by 16")

    @property
    def code(self):
        return _DTYPE_CODE[self.dtype]

    @property
    def storage(self):
        """numpy dtype of the caches."""
        return _NP_STORAGE[self.code]

    @property
    def input_storage(self):
        """numpy dtype of q, k_new and v_new."""
        return _NP_INPUT[self.code]

    def cache_shape(self):
        """Shape of the K cache (and of V, except for INT8)."""
        G, D = self.n_kv_heads, self.head_dim
        if self.dtype == "i8":
            m = self.block_size // 16
            if m == 1:
                return (self.num_blocks, G, 16, D)
            if m > 1:
                return (self.num_blocks, m, G, 16, D)
            return (self.batch, self.max_seq_len // 16, G, 16, D)
        if self.block_size:
            return (self.num_blocks, self.block_size, G, D)
        return (self.batch, self.max_seq_len, G, D)

    def v_cache_shape(self):
        if self.dtype != "i8":
            return self.cache_shape()
        G, D = self.n_kv_heads, self.head_dim
        m = self.block_size // 16
        if m == 1:
            return (self.num_blocks, G, D, 16)
        if m > 1:
            return (self.num_blocks, m, G, D, 16)
        return (self.batch, self.max_seq_len // 16, G, D, 16)

    def _c(self):
        return _Shape(self.batch, self.n_heads, self.n_kv_heads, self.head_dim,
                      self.code, self.block_size, self.max_seq_len, self.num_blocks,
                      self.max_blocks_per_seq)


def theta(i: int, head_dim: int, base: float = 10000.0) -> float:
    """theta_i = base^(-2i/D) ([KVGR] §3)."""
    return _load().kvo_theta(i, head_dim, base)


def round_to_bf16(x: float) -> float:
    """Nearest bf16 value of the fp64 number x, ties to even, one rounding."""
    return _load().kvo_round_to_bf16(float(x))


def bf16_bits(x: float) -> int:
    return int(_load().kvo_bf16_bits(float(x)))


def quantize_i8(x: float, s: float) -> int:
    """INT8 code of x under scale s: nearest integer to x / s in [-127, 127]
    (ties to even, fp64 quotient, saturating; NaN gives 0) ([KVGR] §4.3)."""
    return int(_load().kvo_quantize_i8(float(x), float(s)))


def _scales(geom, k_scale, v_scale):
    if geom.dtype != "i8":
        if k_scale is not None or v_scale is not None:
            raise ValueError("scales are only for INT8 caches")
        return None, None
    G = geom.n_kv_heads
    return (_need(k_scale, np.float32, "k_scale", (G,)), _need(v_scale, np.float32, "v_scale", (G,)))


def rope_rotate(x, pos, base=10000.0, style="interleaved"):
    """R_pos x for every row of an fp64 array [..., D] ([KVGR] §3)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    D = x.shape[-1]
    flat = x.reshape(-1, D)
    out = np.empty_like(flat)
    lib = _load()
    for r in range(flat.shape[0]):
        lib.kvo_rope_rotate(_ptr(flat[r]), _ptr(out[r]), D, float(pos), float(base),
                            _STYLE_CODE[style])
    return out.reshape(x.shape)


def rope_append(geom: Geometry, q, k_new, v_new, k_cache, v_cache, positions,
                block_table=None, base=10000.0, style="interleaved", k_scale=None,
                v_scale=None, n_query=1):
    """Rotate q and k_new at positions[b] and write k_rot, v_new into the caches.

    The caches are modified in place.  Returns q_rot [B, H, D] fp64.
    INT8 caches take the per-head scales ``k_scale``, ``v_scale`` ([G] fp32).
    With ``n_query`` = T > 1 each sequence brings T new tokens (q [B, T, H, D],
    k_new / v_new [B, T, G, D]) for slots positions[b] .. positions[b] + T - 1
    ([OPT] §五, the verification pass); q_rot is then [B, T, H, D].
    Raises ValueError if a position or block id does not exist.
    """
    B, H, G, D = geom.batch, geom.n_heads, geom.n_kv_heads, geom.head_dim
    T = int(n_query)
    st, ist = geom.storage, geom.input_storage
    lead = (B,) if T == 1 else (B, T)
    if q is not None:
        _need(q, ist, "q", (*lead, H, D))
    _need(k_new, ist, "k_new", (*lead, G, D))
    _need(v_new, ist, "v_new", (*lead, G, D))
    _need(k_cache, st, "k_cache", geom.cache_shape())
    _need(v_cache, st, "v_cache", geom.v_cache_shape())
    _need(positions, np.int32, "positions", (B,))
    if geom.block_size:
        _need(block_table, np.int32, "block_table", (B, geom.max_blocks_per_seq))
    ks, vs = _scales(geom, k_scale, v_scale)
    q_rot = np.zeros((*lead, H, D), np.float64)
    sh = geom._c()
    if T > 1:
        rc = _load().kvo_rope_append_mq(ctypes.byref(sh), T, _ptr(q), _ptr(k_new), _ptr(v_new),
                                        _ptr(q_rot), _ptr(k_cache), _ptr(v_cache), _ptr(ks),
                                        _ptr(vs), _ptr(positions), _ptr(block_table),
                                        float(base), _STYLE_CODE[style])
    elif geom.dtype == "i8":
        rc = _load().kvo_rope_append_i8(ctypes.byref(sh), _ptr(q), _ptr(k_new), _ptr(v_new),
                                        _ptr(q_rot), _ptr(k_cache), _ptr(v_cache), _ptr(ks),
                                        _ptr(vs), _ptr(positions), _ptr(block_table),
                                        float(base), _STYLE_CODE[style])
    else:
        rc = _load().kvo_rope_append(ctypes.byref(sh), _ptr(q), _ptr(k_new), _ptr(v_new),
                                     _ptr(q_rot), _ptr(k_cache), _ptr(v_cache),
                                     _ptr(positions), _ptr(block_table), float(base),
                                     _STYLE_CODE[style])
    if rc != 0:
        raise ValueError("position or block id out of range")
    return q_rot


def decode_attn(geom: Geometry, q_rot, k_cache, v_cache, seq_lens, block_table=None,
                scale=None, want_probs=False, n_threads=None, k_scale=None, v_scale=None,
                n_query=1):
    """fp64 attention of every (b, h) query over its first seq_lens[b] tokens.

    Returns (out [B,H,D], lse [B,H]) and, with want_probs, the weights
    [B, H, max_seq_len] (zero past seq_lens[b]).  INT8 caches take their
    per-head scales.  With ``n_query`` = T > 1, q_rot is [B, T, H, D] and
    query t of sequence b attends the tokens j < seq_lens[b] - T + 1 + t;
    out is [B, T, H, D], lse [B, T, H].
    """
    B, H, D = geom.batch, geom.n_heads, geom.head_dim
    T = int(n_query)
    lead = (B,) if T == 1 else (B, T)
    _need(q_rot, np.float64, "q_rot", (*lead, H, D))
    _need(k_cache, geom.storage, "k_cache", geom.cache_shape())
    _need(v_cache, geom.storage, "v_cache", geom.v_cache_shape())
    ks, vs = _scales(geom, k_scale, v_scale)
    _need(seq_lens, np.int32, "seq_lens", (B,))
    if geom.block_size:
        _need(block_table, np.int32, "block_table", (B, geom.max_blocks_per_seq))
    if scale is None:
        scale = 1.0 / np.sqrt(D)  # default 1/sqrt(d_k), d_k = per-head dim ([KVGR] §2.1)
    out = np.zeros((*lead, H, D), np.float64)
    lse = np.zeros((*lead, H), np.float64)
    probs = np.zeros((*lead, H, geom.max_seq_len), np.float64) if want_probs else None
    sh = geom._c()
    rc = _load().kvo_decode_attn_mq(ctypes.byref(sh), T, _ptr(q_rot), _ptr(k_cache),
                                    _ptr(v_cache), _ptr(ks), _ptr(vs), _ptr(seq_lens),
                                    _ptr(block_table), float(scale), _ptr(out), _ptr(lse),
                                    _ptr(probs), n_threads or default_threads())
    if rc != 0:
        raise ValueError("a referenced cache slot does not exist")
    return (out, lse, probs) if want_probs else (out, lse)


def decode_attn_units(geom: Geometry, q_rot, k_cache, v_cache, seq_lens, units,
                      block_table=None, scale=None, n_threads=None, k_scale=None,
                      v_scale=None, n_query=1):
    """As decode_attn, for the listed (b, h) pairs (T > 1: (b, t, h) triples)
    only: returns out [n, D], lse [n]."""
    B, H, D = geom.batch, geom.n_heads, geom.head_dim
    T = int(n_query)
    lead = (B,) if T == 1 else (B, T)
    _need(q_rot, np.float64, "q_rot", (*lead, H, D))
    _need(k_cache, geom.storage, "k_cache", geom.cache_shape())
    _need(v_cache, geom.storage, "v_cache", geom.v_cache_shape())
    ks, vs = _scales(geom, k_scale, v_scale)
    _need(seq_lens, np.int32, "seq_lens", (B,))
    if geom.block_size:
        _need(block_table, np.int32, "block_table", (B, geom.max_blocks_per_seq))
    if T == 1:
        units = np.asarray(units, dtype=np.int32).reshape(-1, 2)
        ub = np.ascontiguousarray(units[:, 0])
        uh = np.ascontiguousarray(units[:, 1])
        if ((ub < 0) | (ub >= B) | (uh < 0) | (uh >= H)).any():
            raise ValueError("unit out of range")
    else:
        units = np.asarray(units, dtype=np.int32).reshape(-1, 3)
        if ((units[:, 0] < 0) | (units[:, 0] >= B) | (units[:, 1] < 0) | (units[:, 1] >= T) |
                (units[:, 2] < 0) | (units[:, 2] >= H)).any():
            raise ValueError("unit out of range")
        ub = np.ascontiguousarray(units[:, 0])
        uh = np.ascontiguousarray(units[:, 1] * H + units[:, 2])
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    n = units.shape[0]
    out = np.zeros((n, D), np.float64)
    lse = np.zeros((n,), np.float64)
    sh = geom._c()
    rc = _load().kvo_decode_attn_units_mq(ctypes.byref(sh), T, _ptr(q_rot), _ptr(k_cache),
                                          _ptr(v_cache), _ptr(ks), _ptr(vs), _ptr(seq_lens),
                                          _ptr(block_table), float(scale), _ptr(ub), _ptr(uh),
                                          n, _ptr(out), _ptr(lse),
                                          n_threads or default_threads())
    if rc != 0:
        raise ValueError("a referenced cache slot does not exist")
    return out, lse


def recent_shape(geom: Geometry, window: int):
    """Shape of a bf16 ring of the ``window`` newest tokens: [B, W, G, D]."""
    return (geom.batch, int(window), geom.n_kv_heads, geom.head_dim)


def rope_append_mixed(geom: Geometry, window, q, k_new, v_new, k_cache, v_cache, k_recent,
                      v_recent, positions, block_table=None, base=10000.0,
                      style="interleaved", k_scale=None, v_scale=None):
    """The append into a mixed-precision cache (module docstring): geom
    describes the INT8 cache; k_recent / v_recent are uint16 bf16 rings
    [B, W, G, D].  Everything is modified in place; returns q_rot [B, H, D]
    fp64.  Raises ValueError if a position or a block id does not exist."""
    if geom.dtype != "i8":
        raise ValueError("the history of a mixed cache is INT8")
    B, H, G, D = geom.batch, geom.n_heads, geom.n_kv_heads, geom.head_dim
    if q is not None:
        _need(q, np.uint16, "q", (B, H, D))
    _need(k_new, np.uint16, "k_new", (B, G, D))
    _need(v_new, np.uint16, "v_new", (B, G, D))
    _need(k_cache, np.int8, "k_cache", geom.cache_shape())
    _need(v_cache, np.int8, "v_cache", geom.v_cache_shape())
    _need(k_recent, np.uint16, "k_recent", recent_shape(geom, window))
    _need(v_recent, np.uint16, "v_recent", recent_shape(geom, window))
    _need(positions, np.int32, "positions", (B,))
    if geom.block_size:
        _need(block_table, np.int32, "block_table", (B, geom.max_blocks_per_seq))
    ks, vs = _scales(geom, k_scale, v_scale)
    q_rot = np.zeros((B, H, D), np.float64)
    rc = _load().kvo_rope_append_mixed(ctypes.byref(geom._c()), int(window), _ptr(q),
                                       _ptr(k_new), _ptr(v_new), _ptr(q_rot), _ptr(k_cache),
                                       _ptr(v_cache), _ptr(ks), _ptr(vs), _ptr(k_recent),
                                       _ptr(v_recent), _ptr(positions), _ptr(block_table),
                                       float(base), _STYLE_CODE[style])
    if rc != 0:
        raise ValueError("position or block id out of range")
    return q_rot


def decode_attn_mixed(geom: Geometry, window, q_rot, k_cache, v_cache, k_recent, v_recent,
                      seq_lens, block_table=None, scale=None, k_scale=None, v_scale=None,
                      units=None, n_threads=None):
    """fp64 attention over a mixed-precision cache: every (b, h), or the
    listed (b, h) pairs; returns (out, lse) of shape [B, H, D], [B, H] or
    [n, D], [n]."""
    if geom.dtype != "i8":
        raise ValueError("the history of a mixed cache is INT8")
    B, H, D = geom.batch, geom.n_heads, geom.head_dim
    _need(q_rot, np.float64, "q_rot", (B, H, D))
    _need(k_cache, np.int8, "k_cache", geom.cache_shape())
    _need(v_cache, np.int8, "v_cache", geom.v_cache_shape())
    _need(k_recent, np.uint16, "k_recent", recent_shape(geom, window))
    _need(v_recent, np.uint16, "v_recent", recent_shape(geom, window))
    _need(seq_lens, np.int32, "seq_lens", (B,))
    if geom.block_size:
        _need(block_table, np.int32, "block_table", (B, geom.max_blocks_per_seq))
    ks, vs = _scales(geom, k_scale, v_scale)
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    ub = uh = None
    if units is None:
        n = B * H
        out = np.zeros((B, H, D), np.float64)
        lse = np.zeros((B, H), np.float64)
    else:
        u = np.asarray(units, dtype=np.int32).reshape(-1, 2)
        if ((u[:, 0] < 0) | (u[:, 0] >= B) | (u[:, 1] < 0) | (u[:, 1] >= H)).any():
            raise ValueError("unit out of range")
        ub, uh = np.ascontiguousarray(u[:, 0]), np.ascontiguousarray(u[:, 1])
        n = u.shape[0]
        out = np.zeros((n, D), np.float64)
        lse = np.zeros((n,), np.float64)
    rc = _load().kvo_decode_attn_mixed(ctypes.byref(geom._c()), int(window), _ptr(q_rot),
                                       _ptr(k_cache), _ptr(v_cache), _ptr(ks), _ptr(vs),
                                       _ptr(k_recent), _ptr(v_recent), _ptr(seq_lens),
                                       _ptr(block_table), float(scale), _ptr(ub), _ptr(uh), n,
                                       _ptr(out), _ptr(lse), n_threads or default_threads())
    if rc != 0:
        raise ValueError("a referenced cache slot does not exist")
    return out, lse
